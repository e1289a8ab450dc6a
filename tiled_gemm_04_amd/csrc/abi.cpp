// C ABI of libtgemm.so: argument validation, kernel selection, launch.
//
// The interface follows the DeepGEMM page, section 1.3 (a plain function a
// framework or an inference engine can call directly) and the linear layer
// Y = X W + b of the GEMM compute-cost page, section 3.1.  Validation happens
// before any HIP call, so a rejected request enqueues nothing and leaves C
// untouched.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tgemm.h"
#include "launch.h"


using tgemm::Bf16Args;
using tgemm::Fp8Args;

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kThinMaxM = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// The largest element offset (rows-1)*ld + cols-1 must stay below 2^62.
bool extent_ok(int64_t rows, int64_t cols, int64_t ld) {
  if (rows == 0 || cols == 0) return true;
  constexpr int64_t kLimit = int64_t{1} << 62;
  if (ld <= 0 || cols > kLimit) return false;
  return rows - 1 <= (kLimit - cols) / ld;
}

int validate_bf16(const void* A, const void* B, const void* bias, const void* C, int64_t M,
                  int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int epilogue,
                  int out_dtype, int algo) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return TGEMM_ERR_INVALID;
  if (epilogue < TGEMM_EPI_NONE || epilogue > TGEMM_EPI_BIAS_GELU_TANH) return TGEMM_ERR_INVALID;
  if (out_dtype != TGEMM_OUT_F32 && out_dtype != TGEMM_OUT_BF16) return TGEMM_ERR_INVALID;
  if (algo < TGEMM_ALGO_AUTO || algo > TGEMM_ALGO_TILED_128x128) return TGEMM_ERR_INVALID;
  if (lda < K || ldb < N || ldc < N) return TGEMM_ERR_INVALID;
  if (lda < 1 || ldb < 1 || ldc < 1) return TGEMM_ERR_INVALID;
  if (!extent_ok(M, K, lda) || !extent_ok(K, N, ldb) || !extent_ok(M, N, ldc))
    return TGEMM_ERR_INVALID;
  if (M == 0 || N == 0) return TGEMM_OK;
  if (C == nullptr) return TGEMM_ERR_INVALID;
  if (K > 0 && (A == nullptr || B == nullptr)) return TGEMM_ERR_INVALID;
  if (epilogue != TGEMM_EPI_NONE && bias == nullptr) return TGEMM_ERR_INVALID;
  if (algo == TGEMM_ALGO_THIN && M > kThinMaxM) return TGEMM_ERR_UNSUPPORTED;
  return TGEMM_OK;
}

// Shape-to-kernel table for the tiled family.  A launch wants at least one
// full round of 256 workgroups (one per compute unit) and few idle units in
// its last round; bigger tiles re-read less and run closer to the MFMA peak,
// but only the part of a tile inside C is useful work (a 256-row tile at
// M = 128 computes half padding).  Score = fill of the rounds x useful
// fraction of the tiles' area x the shape's measured efficiency; checked by
// the offline autotune sweep (tiled_gemm_04_amd/autotune.py).
int pick_tiled_shape(int64_t M, int64_t N) {
  static const double kTileEfficiency[tgemm::kNumTiledShapes] = {1.0, 0.86, 0.62};
  constexpr int64_t kCUs = 256;
  int best = tgemm::kTile128x128;
  double best_score = -1.0;
  for (int s = 0; s < tgemm::kNumTiledShapes; ++s) {
    const tgemm::TiledShapeInfo info = tgemm::tiled_shape_info(s);
    const int64_t tm = (M + info.bm - 1) / info.bm, tn = (N + info.bn - 1) / info.bn;
    const int64_t tiles = tm * tn;
    const int64_t rounds = (tiles + kCUs - 1) / kCUs;
    const double fill = static_cast<double>(tiles) / static_cast<double>(rounds * kCUs);
    const double useful = (static_cast<double>(M) / static_cast<double>(tm * info.bm)) *
                          (static_cast<double>(N) / static_cast<double>(tn * info.bn));
    const double score = fill * useful * kTileEfficiency[s];
    if (score > best_score + 1e-9) {
      best_score = score;
      best = s;
    }
  }
  return best;
}

// Tile shape for the tiled family: fixed by the algo, else the table below.
int tiled_shape_for(int64_t M, int64_t N, int algo) {
  switch (algo) {
    case TGEMM_ALGO_TILED_256x256: return tgemm::kTile256x256;
    case TGEMM_ALGO_TILED_256x128: return tgemm::kTile256x128;
    case TGEMM_ALGO_TILED_128x128: return tgemm::kTile128x128;
    default: return pick_tiled_shape(M, N);
  }
}

bool use_thin(int64_t M, int algo) {
  if (algo == TGEMM_ALGO_THIN) return true;
  if (algo != TGEMM_ALGO_AUTO) return false;  // the tiled family, any tile shape
  return M <= kThinMaxM;
}

// A workspace argument pair: NULL with any size means "none given"; a
// non-NULL workspace must be 16-byte aligned and hold at least `need` bytes.
bool workspace_ok(const void* ws, int64_t bytes, int64_t need) {
  if (ws == nullptr) return true;
  return aligned16(ws) && bytes >= need;
}

int64_t round256(int64_t bytes) { return (bytes + 255) / 256 * 256; }

// Workspace bytes of the small-M bf16 split (0 when the plan does not split
// or the call would not take the thin kernel).
int64_t bf16_ws_bytes(int64_t M, int64_t N, int64_t K, int algo) {
  if (M == 0 || N == 0 || !use_thin(M, algo)) return 0;
  return round256(tgemm::thin_split_bytes(tgemm::thin_split_plan(M, N, K), M, N));
}

int64_t wq_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M == 0 || N == 0) return 0;
  return round256(tgemm::thin_split_bytes(tgemm::wq_split_plan(M, N, K), M, N));
}

// FP8 split workspace: the per-tile counters first (4 bytes each, the
// region rounded up to 256 bytes), then the fp32 partial tiles.
int64_t fp8_counter_bytes(const tgemm::Fp8Split& plan) { return round256(int64_t{4} * plan.split_tiles); }

int64_t fp8_ws_bytes(const tgemm::Fp8Split& plan) {
  if (plan.parts <= 1) return 0;
  return fp8_counter_bytes(plan) + static_cast<int64_t>(tgemm::fp8_split_part_bytes(plan));
}

// Weight-only integer GEMM (bits = 8 or 4): the argument rules of gemm_bf16
// with Q in place of B (row stride in bytes; int4 rows hold two K rows each).
int gemm_weight_only(int bits, const void* X, const void* Q, const float* S, const void* bias,
                     void* C, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                     int epilogue, int out_dtype, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  const int v = validate_bf16(X, Q, bias, C, M, N, K, ldx, ldq, ldc, epilogue, out_dtype,
                              TGEMM_ALGO_AUTO);
  if (v != TGEMM_OK || M == 0 || N == 0) return v;
  if (K > 0 && S == nullptr) return TGEMM_ERR_INVALID;
  if (!tgemm::wq_supported(bits, M, N, K, ldx, ldq)) return TGEMM_ERR_UNSUPPORTED;
  if (!workspace_ok(workspace, workspace_bytes, wq_ws_bytes(M, N, K))) return TGEMM_ERR_INVALID;
  tgemm::W8Args a;
  a.X = static_cast<const uint16_t*>(X);
  a.Q = static_cast<const uint8_t*>(Q);
  a.S = S;
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.ldx = ldx;
  a.ldq = ldq;
  a.ldc = ldc;
  // A lane stores 4 consecutive outputs: 8 bytes of bf16 or 16 bytes of fp32.
  a.vec_c = ((out_dtype == TGEMM_OUT_BF16 ? aligned8(C) : aligned16(C)) && ldc % 4 == 0) ? 1 : 0;
  const hipError_t e = tgemm::launch_wq_thin(bits, a, epilogue, out_dtype == TGEMM_OUT_BF16 ? 1 : 0,
                                             static_cast<hipStream_t>(stream), static_cast<float*>(workspace),
                                             workspace_bytes);
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

// Workspace split of the log-softmax heads: (max, sum exp) pairs first,
// rounded up to 256 bytes, then the fp32 logits when the output is bf16
// (fp32 output holds them in C itself).
tgemm::LsmArgs lsm_args(void* workspace, int64_t M, int64_t N, int out_dtype, void* C, int64_t ldc,
                        int vec_c) {
  tgemm::LsmArgs q;
  q.part = static_cast<float2*>(workspace);
  q.G = static_cast<int>(tgemm::lsm_workgroups(N));
  if (out_dtype == TGEMM_OUT_F32) {
    q.logits = static_cast<float*>(C);
    q.ldl = ldc;
    q.vec_l = vec_c;
  } else {
    q.logits = reinterpret_cast<float*>(static_cast<char*>(workspace) + (M * q.G * 8 + 255) / 256 * 256);
    q.ldl = N;
    q.vec_l = aligned16(q.logits) ? 1 : 0;
  }
  return q;
}

int64_t lsm_workspace_bytes(int64_t M, int64_t N, int out_dtype) {
  const int64_t pairs = (M * tgemm::lsm_workgroups(N) * 8 + 255) / 256 * 256;
  return pairs + (out_dtype == TGEMM_OUT_BF16 ? M * N * 4 : 0);
}

int gemm_wq_logsoftmax(int bits, const void* X, const void* Q, const float* S, const void* bias,
                       void* C, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                       int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (M > 0 && N == 0) return TGEMM_ERR_INVALID;  // no distribution over zero columns
  const int v = validate_bf16(X, Q, bias, C, M, N, K, ldx, ldq, ldc, TGEMM_EPI_NONE, out_dtype,
                              TGEMM_ALGO_AUTO);
  if (v != TGEMM_OK || M == 0) return v;
  if (K > 0 && S == nullptr) return TGEMM_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < lsm_workspace_bytes(M, N, out_dtype))
    return TGEMM_ERR_INVALID;
  if (!tgemm::wq_supported(bits, M, N, K, ldx, ldq)) return TGEMM_ERR_UNSUPPORTED;
  tgemm::W8Args a;
  a.X = static_cast<const uint16_t*>(X);
  a.Q = static_cast<const uint8_t*>(Q);
  a.S = S;
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.ldx = ldx;
  a.ldq = ldq;
  a.ldc = ldc;
  const int64_t out_align = out_dtype == TGEMM_OUT_BF16 ? 8 : 4;
  a.vec_c = (aligned16(C) && ldc % out_align == 0) ? 1 : 0;
  const tgemm::LsmArgs q = lsm_args(workspace, M, N, out_dtype, C, ldc, a.vec_c);
  const hipError_t e = tgemm::launch_wq_thin_lsm(bits, a, q, out_dtype == TGEMM_OUT_BF16 ? 1 : 0,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

const char* weight_only_name(int bits, int64_t M, int64_t N, int64_t K, int with_workspace) {
  if (M < 1 || N < 1 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return nullptr;
  if (!tgemm::wq_supported(bits, M, N, K, K, N)) return nullptr;
  const bool split = with_workspace != 0 && tgemm::wq_split_plan(M, N, K).S > 1;
  return tgemm::wq_kernel_name(bits, static_cast<int>(M), split);
}

int quantize_fp8(const void* X, void* Q, float* S, int64_t rows, int64_t cols, int64_t ldx,
                 void* stream, bool blocks) {
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return TGEMM_ERR_INVALID;
  if (rows == 0 || cols == 0) return TGEMM_OK;
  if (X == nullptr || Q == nullptr || S == nullptr || ldx < cols) return TGEMM_ERR_INVALID;
  if (!extent_ok(rows, cols, ldx) || !extent_ok(rows, cols, cols)) return TGEMM_ERR_INVALID;
  tgemm::QuantArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.Q = static_cast<uint8_t*>(Q);
  a.S = S;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.groups_per_row = (cols + 127) / 128;
  a.vec_in = (aligned16(X) && ldx % 8 == 0) ? 1 : 0;
  a.vec_out = (aligned8(Q) && cols % 8 == 0) ? 1 : 0;
  const hipError_t e = blocks ? tgemm::launch_quant_fp8_128x128(a, static_cast<hipStream_t>(stream))
                              : tgemm::launch_quant_fp8_1x128(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidConfiguration) return TGEMM_ERR_UNSUPPORTED;
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

// FP8 block-scaled GEMM with B given as [K, N] (bt false) or [N, K] (bt
// true); the split plan and its workspace as gemm_fp8_blockscaled_ex
// documents (no workspace: unsplit).
int fp8_call(const void* A, const float* sA, const void* B, const float* sB, void* C, int64_t M,
             int64_t N, int64_t K, int split_parts, bool bt, void* workspace, int64_t workspace_bytes,
             void* stream) {
  if (split_parts < 0 || split_parts > tgemm::kFp8MaxParts) return TGEMM_ERR_INVALID;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return TGEMM_ERR_INVALID;
  if (M == 0 || N == 0) return TGEMM_OK;
  if (C == nullptr) return TGEMM_ERR_INVALID;
  if (K > 0 && (A == nullptr || B == nullptr || sA == nullptr || sB == nullptr))
    return TGEMM_ERR_INVALID;
  if (!extent_ok(M, K, K) || !extent_ok(M, N, N)) return TGEMM_ERR_INVALID;
  if (bt ? !extent_ok(N, K, K) : !extent_ok(K, N, N)) return TGEMM_ERR_INVALID;
  if (bt && !tgemm::fp8_nt_ok(M, N, K)) return TGEMM_ERR_UNSUPPORTED;
  const tgemm::Fp8Split plan =
      workspace == nullptr ? tgemm::Fp8Split{0, 0, 1}
                           : tgemm::fp8_split_plan(M, N, K, tgemm::device_cus(), split_parts);
  if (!workspace_ok(workspace, workspace_bytes, fp8_ws_bytes(plan))) return TGEMM_ERR_INVALID;

  Fp8Args a;
  a.A = static_cast<const uint8_t*>(A);
  a.sA = sA;
  a.B = static_cast<const uint8_t*>(B);
  a.sB = sB;
  a.C = static_cast<uint16_t*>(C);
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.G = static_cast<int>((K + 127) / 128);
  a.H = static_cast<int>((N + 127) / 128);
  a.vec_a = (aligned16(A) && K % 16 == 0) ? 1 : 0;
  a.vec_b = bt ? a.vec_a : ((aligned8(B) && N % 8 == 0) ? 1 : 0);
  a.vec_c = (aligned16(C) && N % 8 == 0) ? 1 : 0;
  a.bt = bt ? 1 : 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // Split the tiles along K when they leave most compute units idle: the
  // counters open the workspace, the partial tiles follow them.
  void* part = nullptr;
  uint32_t* count = nullptr;
  if (plan.parts > 1) {
    count = static_cast<uint32_t*>(workspace);
    part = static_cast<char*>(workspace) + fp8_counter_bytes(plan);
  }
  // Automatic mode also cuts a sparse last round of tiles into halves.
  const hipError_t e = tgemm::launch_fp8_blockscaled(a, plan, part, count, split_parts == 0, s);
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

}  // namespace

namespace tgemm {

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace tgemm

extern "C" {

int gemm_bf16_ex(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                 int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, int out_dtype,
                 int algo, void* workspace, int64_t workspace_bytes, void* stream) {
  const int st = validate_bf16(A, B, bias, C, M, N, K, lda, ldb, ldc, epilogue, out_dtype, algo);
  if (st != TGEMM_OK) return st;
  if (M == 0 || N == 0) return TGEMM_OK;
  if (!workspace_ok(workspace, workspace_bytes, bf16_ws_bytes(M, N, K, algo))) return TGEMM_ERR_INVALID;

  Bf16Args a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.vec_a = (K == 0 || (aligned16(A) && lda % 8 == 0)) ? 1 : 0;
  a.vec_b = (K == 0 || (aligned16(B) && ldb % 8 == 0)) ? 1 : 0;
  const int64_t out_align = out_dtype == TGEMM_OUT_BF16 ? 8 : 4;
  a.vec_c = (aligned16(C) && ldc % out_align == 0) ? 1 : 0;

  const int out_bf16 = out_dtype == TGEMM_OUT_BF16 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_thin(M, algo)) {
    e = tgemm::launch_bf16_thin(a, epilogue, out_bf16, s, static_cast<float*>(workspace), workspace_bytes);
  } else {
    e = tgemm::launch_bf16_tiled(a, tiled_shape_for(M, N, algo), epilogue, out_bf16, s);
  }
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int gemm_bf16_noalloc(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                      int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, int out_dtype,
                      int algo, void* stream) {
  static_assert(tgemm::kNoAllocScratchBytes == TGEMM_NOALLOC_SCRATCH_BYTES, "header and library agree");
  const int st = validate_bf16(A, B, bias, C, M, N, K, lda, ldb, ldc, epilogue, out_dtype, algo);
  if (st != TGEMM_OK) return st;
  if (M == 0 || N == 0) return TGEMM_OK;
  const int64_t need = bf16_ws_bytes(M, N, K, algo);
  if (need > tgemm::kNoAllocScratchBytes) return TGEMM_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && tgemm::noalloc_scratch(&ws) != hipSuccess) return TGEMM_ERR_LAUNCH;
  return gemm_bf16_ex(A, B, bias, C, M, N, K, lda, ldb, ldc, epilogue, out_dtype, algo, ws, need, stream);
}

int64_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K, int algo) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
  if (algo < TGEMM_ALGO_AUTO || algo > TGEMM_ALGO_TILED_128x128) return -1;
  return bf16_ws_bytes(M, N, K, algo);
}

int gemm_bf16_quant_fp8(const void* A, const void* B, const void* bias, void* Q, float* S,
                        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int epilogue,
                        int algo, void* stream) {
  // Q is [M, N] bytes, packed: checked as C with ldc = N.
  const int st = validate_bf16(A, B, bias, Q, M, N, K, lda, ldb, N > 0 ? N : 1, epilogue,
                               TGEMM_OUT_BF16, algo);
  if (st != TGEMM_OK) return st;
  if (algo == TGEMM_ALGO_THIN) return TGEMM_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return TGEMM_OK;
  if (S == nullptr) return TGEMM_ERR_INVALID;
  Bf16Args a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = Q;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = N;
  a.vec_a = (K == 0 || (aligned16(A) && lda % 8 == 0)) ? 1 : 0;
  a.vec_b = (K == 0 || (aligned16(B) && ldb % 8 == 0)) ? 1 : 0;
  a.vec_c = (aligned8(Q) && N % 8 == 0) ? 1 : 0;
  a.qscale = S;
  const int shape = tiled_shape_for(M, N, algo);
  if (!tgemm::bf16_direct_ok(a, shape)) return TGEMM_ERR_UNSUPPORTED;
  const hipError_t e = tgemm::launch_bf16_tiled_q8(a, shape, epilogue, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int gemm_bf16_nt(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
                 int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, int out_dtype,
                 void* stream) {
  // validate_bf16 checks B as [K, N] with ldb >= N; here B is [N, K].
  const int st = validate_bf16(A, B, bias, C, M, N, K, lda, N > 0 ? N : 1, ldc, epilogue, out_dtype,
                               TGEMM_ALGO_AUTO);
  if (st != TGEMM_OK) return st;
  if (ldb < K || ldb < 1 || !extent_ok(N, K, ldb)) return TGEMM_ERR_INVALID;
  if (M == 0 || N == 0) return TGEMM_OK;
  Bf16Args a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.vec_a = (K == 0 || (aligned16(A) && lda % 8 == 0)) ? 1 : 0;
  a.vec_b = (K == 0 || (aligned16(B) && ldb % 8 == 0)) ? 1 : 0;
  const int64_t out_align = out_dtype == TGEMM_OUT_BF16 ? 8 : 4;
  a.vec_c = (aligned16(C) && ldc % out_align == 0) ? 1 : 0;
  const int out_bf16 = out_dtype == TGEMM_OUT_BF16 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_thin(M, TGEMM_ALGO_AUTO) && tgemm::thin_nt_ok(a)) {
    e = tgemm::launch_bf16_thin_nt(a, epilogue, out_bf16, s);
  } else {
    const int shape = pick_tiled_shape(M, N);
    if (!tgemm::bf16_bt_direct_ok(a, shape)) return TGEMM_ERR_UNSUPPORTED;
    e = tgemm::launch_bf16_tiled_bt(a, shape, epilogue, out_bf16, s);
  }
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

const char* gemm_bf16_nt_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return nullptr;
  if (K % 8 != 0) return nullptr;
  if (use_thin(M, TGEMM_ALGO_AUTO)) {
    static const char* const kThin[4] = {"tgemm_bf16_thin_nt_m16", "tgemm_bf16_thin_nt_m32",
                                         "tgemm_bf16_thin_nt_m48", "tgemm_bf16_thin_nt_m64"};
    return kThin[(M - 1) / 16];
  }
  static const char* const kNames[tgemm::kNumTiledShapes] = {
      "tgemm_bf16_tiled_bt_256x256x32", "tgemm_bf16_tiled_bt_256x128x64", "tgemm_bf16_tiled_bt_128x128x64"};
  const int shape = pick_tiled_shape(M, N);
  return shape >= 0 && shape < tgemm::kNumTiledShapes ? kNames[shape] : nullptr;
}

int gemm_bf16_strided_batched(const void* A, const void* B, const void* bias, void* C, int64_t M,
                              int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                              int64_t stride_a, int64_t stride_b, int64_t stride_c, int64_t batch,
                              int b_layout, int epilogue, int out_dtype, void* stream) {
  if (b_layout != TGEMM_B_KN && b_layout != TGEMM_B_NK) return TGEMM_ERR_INVALID;
  const bool nk = b_layout == TGEMM_B_NK;
  // One problem's rules (B as [K, N] or [N, K]).
  const int st = validate_bf16(A, B, bias, C, M, N, K, lda, nk ? (N > 0 ? N : 1) : ldb, ldc, epilogue,
                               out_dtype, TGEMM_ALGO_AUTO);
  if (st != TGEMM_OK) return st;
  if (nk && (ldb < K || ldb < 1 || !extent_ok(N, K, ldb))) return TGEMM_ERR_INVALID;
  if (batch < 0 || stride_a < 0 || stride_b < 0 || stride_c < 0) return TGEMM_ERR_INVALID;
  if (batch == 0 || M == 0 || N == 0) return TGEMM_OK;
  // Whole-batch extents, and no two problems writing the same output.
  constexpr int64_t kLimit = int64_t{1} << 62;
  const int64_t ext_a = (M - 1) * lda + K, ext_b = nk ? (N - 1) * ldb + K : (K - 1) * ldb + N;
  const int64_t ext_c = (M - 1) * ldc + N;
  auto fits = [&](int64_t stride, int64_t ext) {
    return stride == 0 || batch - 1 <= (kLimit - ext) / stride;
  };
  if (!fits(stride_a, K > 0 ? ext_a : 0) || !fits(stride_b, K > 0 ? ext_b : 0) || !fits(stride_c, ext_c))
    return TGEMM_ERR_INVALID;
  if (batch > 1 && stride_c < ext_c) return TGEMM_ERR_INVALID;
  if (batch > 65535) return TGEMM_ERR_UNSUPPORTED;

  Bf16Args a;
  a.A = static_cast<const uint16_t*>(A);
  a.B = static_cast<const uint16_t*>(B);
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.sa = stride_a;
  a.sb = stride_b;
  a.sc = stride_c;
  a.batch = static_cast<int>(batch);
  // Vector paths need every problem's base aligned like the first one's.
  const bool multi = batch > 1;
  a.vec_a = (K == 0 || (aligned16(A) && lda % 8 == 0 && (!multi || stride_a % 8 == 0))) ? 1 : 0;
  a.vec_b = (K == 0 || (aligned16(B) && ldb % 8 == 0 && (!multi || stride_b % 8 == 0))) ? 1 : 0;
  const int64_t out_align = out_dtype == TGEMM_OUT_BF16 ? 8 : 4;
  a.vec_c = (aligned16(C) && ldc % out_align == 0 && (!multi || stride_c % out_align == 0)) ? 1 : 0;

  const int out_bf16 = out_dtype == TGEMM_OUT_BF16 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (nk) {
    if (use_thin(M, TGEMM_ALGO_AUTO) && tgemm::thin_nt_ok(a)) {
      e = tgemm::launch_bf16_thin_nt(a, epilogue, out_bf16, s);
    } else {
      const int shape = pick_tiled_shape(M, N);
      if (!tgemm::bf16_bt_direct_ok(a, shape)) return TGEMM_ERR_UNSUPPORTED;
      e = tgemm::launch_bf16_tiled_bt(a, shape, epilogue, out_bf16, s);
    }
  } else if (use_thin(M, TGEMM_ALGO_AUTO)) {
    e = tgemm::launch_bf16_thin(a, epilogue, out_bf16, s);
  } else {
    e = tgemm::launch_bf16_tiled(a, pick_tiled_shape(M, N), epilogue, out_bf16, s);
  }
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int gemm_bf16(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N,
              int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int epilogue, int out_dtype,
              void* stream) {
  return gemm_bf16_ex(A, B, bias, C, M, N, K, lda, ldb, ldc, epilogue, out_dtype,
                      TGEMM_ALGO_AUTO, nullptr, 0, stream);
}

int64_t gemm_logsoftmax_workspace_size(int64_t M, int64_t N, int out_dtype) {
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return -1;
  if (out_dtype != TGEMM_OUT_F32 && out_dtype != TGEMM_OUT_BF16) return -1;
  return lsm_workspace_bytes(M, N, out_dtype);
}

int gemm_bf16_w8_logsoftmax(const void* X, const void* Q, const float* S, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                            int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_wq_logsoftmax(8, X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, out_dtype, workspace,
                            workspace_bytes, stream);
}

int gemm_bf16_w4_logsoftmax(const void* X, const void* Q, const float* S, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                            int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_wq_logsoftmax(4, X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, out_dtype, workspace,
                            workspace_bytes, stream);
}

int gemm_bf16_logsoftmax(const void* X, const void* W, const void* bias, void* C, int64_t M,
                         int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldc, int out_dtype,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (M > 0 && N == 0) return TGEMM_ERR_INVALID;  // no distribution over zero columns
  const int st = validate_bf16(X, W, bias, C, M, N, K, ldx, ldw, ldc, TGEMM_EPI_NONE, out_dtype,
                               TGEMM_ALGO_AUTO);
  if (st != TGEMM_OK || M == 0) return st;
  if (workspace == nullptr || workspace_bytes < gemm_logsoftmax_workspace_size(M, N, out_dtype))
    return TGEMM_ERR_INVALID;
  Bf16Args a;
  a.A = static_cast<const uint16_t*>(X);
  a.B = static_cast<const uint16_t*>(W);
  a.bias = static_cast<const uint16_t*>(bias);
  a.C = C;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.lda = ldx;
  a.ldb = ldw;
  a.ldc = ldc;
  a.vec_a = (K == 0 || (aligned16(X) && ldx % 8 == 0)) ? 1 : 0;
  a.vec_b = (K == 0 || (aligned16(W) && ldw % 8 == 0)) ? 1 : 0;
  const int64_t out_align = out_dtype == TGEMM_OUT_BF16 ? 8 : 4;
  a.vec_c = (aligned16(C) && ldc % out_align == 0) ? 1 : 0;
  if (!tgemm::lsm_direct_ok(a)) return TGEMM_ERR_UNSUPPORTED;
  const tgemm::LsmArgs q = lsm_args(workspace, M, N, out_dtype, C, ldc, a.vec_c);
  const hipError_t e = tgemm::launch_bf16_thin_lsm(a, q, out_dtype == TGEMM_OUT_BF16 ? 1 : 0,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int gemm_fp8_blockscaled(const void* A, const float* sA, const void* B, const float* sB, void* C,
                         int64_t M, int64_t N, int64_t K, void* stream) {
  return fp8_call(A, sA, B, sB, C, M, N, K, 0, false, nullptr, 0, stream);
}

int gemm_fp8_blockscaled_ex(const void* A, const float* sA, const void* B, const float* sB, void* C,
                            int64_t M, int64_t N, int64_t K, int split_parts, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  return fp8_call(A, sA, B, sB, C, M, N, K, split_parts, false, workspace, workspace_bytes, stream);
}

int64_t gemm_fp8_workspace_size(int64_t M, int64_t N, int64_t K, int split_parts) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
  if (split_parts < 0 || split_parts > tgemm::kFp8MaxParts) return -1;
  if (M == 0 || N == 0) return 0;
  return fp8_ws_bytes(tgemm::fp8_split_plan(M, N, K, tgemm::device_cus(), split_parts));
}

int gemm_fp8_blockscaled_nt(const void* A, const float* sA, const void* Bt, const float* sB, void* C,
                            int64_t M, int64_t N, int64_t K, void* stream) {
  return fp8_call(A, sA, Bt, sB, C, M, N, K, 0, true, nullptr, 0, stream);
}

int gemm_bf16_w8(const void* X, const void* Q, const float* S, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                 int epilogue, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_weight_only(8, X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, epilogue, out_dtype, workspace,
                          workspace_bytes, stream);
}

int gemm_bf16_w4(const void* X, const void* Q, const float* S, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                 int epilogue, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_weight_only(4, X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, epilogue, out_dtype, workspace,
                          workspace_bytes, stream);
}

int64_t gemm_wq_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
  return wq_ws_bytes(M, N, K);
}

const char* gemm_w8_kernel_name(int64_t M, int64_t N, int64_t K, int with_workspace) {
  return weight_only_name(8, M, N, K, with_workspace);
}

const char* gemm_w4_kernel_name(int64_t M, int64_t N, int64_t K, int with_workspace) {
  return weight_only_name(4, M, N, K, with_workspace);
}

int quantize_fp8_1x128(const void* X, void* Q, float* S, int64_t M, int64_t K, int64_t ldx,
                       void* stream) {
  return quantize_fp8(X, Q, S, M, K, ldx, stream, false);
}

int quantize_fp8_128x128(const void* W, void* Q, float* S, int64_t K, int64_t N, int64_t ldw,
                         void* stream) {
  return quantize_fp8(W, Q, S, K, N, ldw, stream, true);
}

const char* gemm_bf16_kernel_name(int64_t M, int64_t N, int64_t K, int epilogue, int out_dtype,
                                  int algo, int with_workspace) {
  // Pointers play no part in the choice; pass dummies so only sizes are checked.
  static const int kDummy = 0;
  const void* d = &kDummy;
  if (validate_bf16(d, d, d, d, M, N, K, K > 0 ? K : 1, N > 0 ? N : 1, N > 0 ? N : 1, epilogue,
                    out_dtype, algo) != TGEMM_OK)
    return nullptr;
  if (use_thin(M, algo))
    return tgemm::thin_kernel_name(static_cast<int>(M),
                                   with_workspace != 0 && tgemm::thin_split_plan(M, N, K).S > 1 && K % 8 == 0 &&
                                       N % 8 == 0);
  return tgemm::tiled_shape_info(tiled_shape_for(M, N, algo)).name;
}

int gemm_fp8_split_plan(int64_t M, int64_t N, int64_t K, int cus, int split_parts, int* whole,
                        int* split_tiles, int* parts) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || cus < 0 ||
      split_parts < 0 || split_parts > tgemm::kFp8MaxParts || whole == nullptr ||
      split_tiles == nullptr || parts == nullptr)
    return TGEMM_ERR_INVALID;
  const tgemm::Fp8Split plan = tgemm::fp8_split_plan(M, N, K, cus, split_parts);
  *whole = plan.whole;
  *split_tiles = plan.split_tiles;
  *parts = plan.parts;
  return TGEMM_OK;
}

int64_t gemm_probe_out_elems(int probe) {
  const int cus = tgemm::device_cus();
  if (cus <= 0) return -1;
  if (probe == TGEMM_PROBE_MFMA_BF16 || probe == TGEMM_PROBE_MFMA_FP8) return tgemm::probe_mfma_threads(cus);
  if (probe == TGEMM_PROBE_STREAM_READ) return tgemm::probe_stream_threads(cus);
  return -1;
}

double gemm_probe_mfma_flop(int probe, int64_t iters) {
  const int cus = tgemm::device_cus();
  if (cus <= 0 || iters < 0) return -1.0;
  // 32 MFMAs per wave and iteration: 32x32x16 bf16 = 32768 FLOP, 16x16x128 fp8 = 65536.
  const double per = probe == TGEMM_PROBE_MFMA_BF16 ? 32768.0 : probe == TGEMM_PROBE_MFMA_FP8 ? 65536.0 : -1.0;
  if (per < 0) return -1.0;
  return static_cast<double>(tgemm::probe_mfma_threads(cus) / 64) * 32.0 * per * static_cast<double>(iters);
}

int gemm_probe_mfma(int probe, int64_t iters, float* out, int64_t out_elems, uint64_t seed, void* stream) {
  if (probe != TGEMM_PROBE_MFMA_BF16 && probe != TGEMM_PROBE_MFMA_FP8) return TGEMM_ERR_INVALID;
  if (iters < 0 || iters > 0x7fffffff || out == nullptr) return TGEMM_ERR_INVALID;
  const int64_t need = gemm_probe_out_elems(probe);
  if (need < 0) return TGEMM_ERR_UNSUPPORTED;
  if (out_elems < need) return TGEMM_ERR_INVALID;
  const hipError_t e = tgemm::launch_probe_mfma(probe == TGEMM_PROBE_MFMA_BF16 ? 0 : 1, tgemm::device_cus(),
                                                static_cast<int>(iters), seed, out,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int gemm_probe_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t out_elems, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || out == nullptr) return TGEMM_ERR_INVALID;
  if (bytes > 0 && (src == nullptr || !aligned16(src))) return TGEMM_ERR_INVALID;
  const int64_t need = gemm_probe_out_elems(TGEMM_PROBE_STREAM_READ);
  if (need < 0) return TGEMM_ERR_UNSUPPORTED;
  if (out_elems < need) return TGEMM_ERR_INVALID;
  const hipError_t e = tgemm::launch_probe_stream_read(src, bytes / 16, tgemm::device_cus(), out,
                                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

const char* gemm_fp8_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return nullptr;
  return tgemm::fp8_kernel_name(M, N, K);
}

const char* gemm_status_string(int status) {
  switch (status) {
    case TGEMM_OK: return "ok";
    case TGEMM_ERR_INVALID: return "invalid argument";
    case TGEMM_ERR_UNSUPPORTED: return "unsupported request";
    case TGEMM_ERR_LAUNCH: return "kernel launch failed";
    case TGEMM_ERR_SCRATCH:
      return "request needs more device scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int gemm_abi_version(void) { return TGEMM_ABI_VERSION; }

}  // extern "C"
