// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

// Problem description for the bf16 kernels.  Sizes are validated by the ABI
// layer (each below 2^31); strides are in elements.
struct Bf16Args {
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* bias;
  void* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int vec_a;  // 1: A rows may be read with 16-byte loads (aligned base, lda % 8 == 0)
  int vec_b;  // 1: same for B
  int vec_c;  // 1: C rows may be written with 16-byte stores
  // Strided batch: problem z (grid y) reads A + z*sa, B + z*sb and writes
  // C + z*sc (elements); a single problem has batch 1.
  int64_t sa = 0, sb = 0, sc = 0;
  int batch = 1;
  // Quantising epilogue only: C holds e4m3fn codes (row stride ldc bytes)
  // and qscale the fp32 scales [M, ceil(N/128)], packed.
  float* qscale = nullptr;
};

// Moves p to problem blockIdx.y of a strided batch (C elements of
// out_bytes bytes).
__device__ __forceinline__ void apply_batch(Bf16Args& p, int out_bytes) {
  const int64_t z = blockIdx.y;
  p.A += z * p.sa;
  p.B += z * p.sb;
  p.C = static_cast<char*>(p.C) + z * p.sc * out_bytes;
}

struct Fp8Args {
  const uint8_t* A;
  const float* sA;
  const uint8_t* B;
  const float* sB;
  uint16_t* C;
  int M, N, K;
  int G;      // ceil(K / 128): A-scale columns, B-scale rows
  int H;      // ceil(N / 128): B-scale columns
  int vec_a;  // 1: A rows are 16-byte aligned (K % 16 == 0 and aligned base)
  int vec_b;  // 1: B rows are 8-byte aligned (N % 8 == 0 and aligned base)
  int vec_c;  // 1: C rows may be written with 16-byte stores (N % 8 == 0, aligned base)
  int bt = 0;  // 1: B is given as [N, K] (K-contiguous rows, packed)
};

// FP8 quantiser problem: bf16 X [rows, cols] (row stride ldx) -> e4m3fn
// codes Q [rows, cols] (packed) and fp32 scales S [.., groups_per_row].
struct QuantArgs {
  const uint16_t* X;
  uint8_t* Q;
  float* S;
  int64_t rows, cols, ldx;
  int64_t groups_per_row;  // ceil(cols / 128)
  int vec_in;   // 1: X rows may be read with 16-byte loads (aligned base, ldx % 8 == 0)
  int vec_out;  // 1: Q rows may be written with 8-byte stores (aligned base, cols % 8 == 0)
};

// Weight-only integer GEMM: bf16 X [M, K] (row stride ldx) times integer
// codes Q (int8: [K, N]; int4: [K/2, N], two codes per byte along K; row
// stride ldq bytes) with fp32 scales S [ceil(K/128), N] (packed), + bias,
// epilogue, into C [M, N] (row stride ldc).
struct W8Args {
  const uint16_t* X;
  const uint8_t* Q;
  const float* S;
  const uint16_t* bias;
  void* C;
  int M, N, K;
  int64_t ldx, ldq, ldc;
  int vec_c;  // 1: C rows may be written with 8- / 16-byte stores
};

// Tiled bf16 kernel shapes (BM x BN output tile, 4 waves).
enum TiledShape { kTile256x256 = 0, kTile256x128 = 1, kTile128x128 = 2, kNumTiledShapes = 3 };

struct TiledShapeInfo {
  int bm, bn;
  const char* name;
};
TiledShapeInfo tiled_shape_info(int shape);

// Each returns hipSuccess or the launch error.
hipError_t launch_bf16_tiled(const Bf16Args& a, int shape, int epilogue, int out_bf16,
                             hipStream_t stream);
// B given as [N, K] (K-contiguous, row stride ldb); hipErrorInvalidValue
// when the operands do not meet bf16_bt_direct_ok.
hipError_t launch_bf16_tiled_bt(const Bf16Args& a, int shape, int epilogue, int out_bf16,
                                hipStream_t stream);
bool bf16_bt_direct_ok(const Bf16Args& a, int shape);
bool bf16_direct_ok(const Bf16Args& a, int shape);
// The tiled kernel with a quantising epilogue: epilogue(A.B + bias) rounded
// to bf16, then 1 x 128 FP8 codes into C (bytes) and scales into qscale.
// hipErrorInvalidValue when the operands do not meet bf16_direct_ok.
hipError_t launch_bf16_tiled_q8(const Bf16Args& a, int shape, int epilogue, hipStream_t stream);
// Small-M kernel for B given as [N, K] (M <= 64, aligned operands).
hipError_t launch_bf16_thin_nt(const Bf16Args& a, int epilogue, int out_bf16, hipStream_t stream);
bool thin_nt_ok(const Bf16Args& a);
// Register-staged kernel for operands the direct-to-LDS kernel cannot take.
hipError_t launch_bf16_general(const Bf16Args& a, int shape, int epilogue, int out_bf16,
                               hipStream_t stream);
// Small-M kernel.  part / part_bytes: caller workspace for the split-K
// partials (nullptr: never split); the split runs when the plan asks for
// one and part_bytes >= thin_split_bytes(plan, M, N).
hipError_t launch_bf16_thin(const Bf16Args& a, int epilogue, int out_bf16, hipStream_t stream,
                            float* part = nullptr, int64_t part_bytes = 0);
// Split-K for the thin kernel: S chunks of ktc slices (S == 1: no split).
struct ThinSplit {
  int S;
  int ktc;
};
ThinSplit thin_split_plan(int64_t M, int64_t N, int64_t K);
// Bytes of fp32 partials a split plan writes: S * M * N * 4 (0 for S == 1).
int64_t thin_split_bytes(const ThinSplit& plan, int64_t M, int64_t N);
// The operands the direct-to-LDS thin kernel (and its split) takes.
bool thin_direct_ok(const Bf16Args& a);
// part: S * M * N fp32 of workspace.
hipError_t launch_bf16_thin_splitk(const Bf16Args& a, const ThinSplit& plan, float* part, int epilogue,
                                   int out_bf16, hipStream_t stream);
// C = epilogue(sum over s < S of part[s] + bias), summed in order of s and
// rounded once; reads a.M, a.N, a.bias, a.C, a.ldc and a.vec_c only.
hipError_t launch_splitk_reduce(const Bf16Args& a, const float* part, int S, int epilogue, int out_bf16,
                                hipStream_t stream);
// Compute units of the current device (0 if unknown).
int device_cus();
// Size of the fixed device scratch of the allocation-free split entry point,
// and its address on the current device (looked up once per device).
constexpr int64_t kNoAllocScratchBytes = int64_t{32} << 20;
hipError_t noalloc_scratch(void** ptr);
// Register-transposing thin kernel for operands the direct-to-LDS one cannot take.
hipError_t launch_bf16_thin_general(const Bf16Args& a, int epilogue, int out_bf16,
                                    hipStream_t stream);
// Tile split of the direct FP8 kernel: `whole` tiles done whole, the last
// round's `split_tiles` tiles in `parts` K ranges each (parts == 1: none).
struct Fp8Split {
  int whole;
  int split_tiles;
  int parts;
};
constexpr int kFp8MaxParts = 8;
constexpr int kFp8MaxSplitTiles = 4096;
// forced_parts: 0 automatic (split only a grid that keeps at most a quarter
// of the compute units busy, at least eight scale groups per part); 1 never;
// 2 .. kFp8MaxParts split the last round's tiles into that many parts (at
// most one per scale group).
Fp8Split fp8_split_plan(int64_t M, int64_t N, int64_t K, int cus, int forced_parts);
size_t fp8_split_part_bytes(const Fp8Split& plan);
// part: fp8_split_part_bytes(plan) of workspace; count: plan.split_tiles
// counters that are zero on entry (and again on exit).  Either NULL: no split.
// halves (without a split): the last round's tiles run as 128-row halves
// when fp8_tail_halves says so (bit-identical results).
hipError_t launch_fp8_blockscaled(const Fp8Args& a, const Fp8Split& plan, void* part,
                                  uint32_t* count, bool halves, hipStream_t stream);
// Tiles of the last round that run as two 128-row halves each: all of them
// when they would occupy at most half of `cus` compute units, else none.
int fp8_tail_halves(int64_t tiles, int cus);
// Register-staged kernel for FP8 operands the direct-to-LDS kernel cannot take.
hipError_t launch_fp8_general(const Fp8Args& a, hipStream_t stream);

// bits: 8 or 4 (the code width).  part / part_bytes: caller workspace for
// the split-K partials (nullptr: never split), as launch_bf16_thin.
hipError_t launch_wq_thin(int bits, const W8Args& a, int epilogue, int out_bf16, hipStream_t stream,
                          float* part = nullptr, int64_t part_bytes = 0);
// Split-K plan of the integer-weight kernel (chunks of whole 128-row scale
// groups; the same for int8 and int4); S == 1: no split.
ThinSplit wq_split_plan(int64_t M, int64_t N, int64_t K);
bool wq_supported(int bits, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq);
// split: the name of the split-K pair (kernel + reduction).
const char* wq_kernel_name(int bits, int M, bool split);
// Thin-M GEMM + bias + row log-softmax, in two passes: the GEMM kernel
// writes fp32 logits (row stride ldl) and per-stripe (max, sum exp) pairs
// part [M, G] (G = lsm_workgroups(N)); the second kernel merges each row's
// pairs and writes logits - lse into C.
struct LsmArgs {
  float2* part;
  float* logits;  // C itself for fp32 output, else workspace
  int64_t ldl;
  int G;
  int vec_l;  // 1: logit rows may be read and written with 16-byte accesses
};
hipError_t launch_bf16_thin_lsm(const Bf16Args& a, const LsmArgs& q, int out_bf16, hipStream_t stream);
// Pass 2 of the log-softmax heads: merge each row's G pairs, write y - lse.
hipError_t launch_lsm_normalize(const LsmArgs& q, void* C, int64_t ldc, int M, int N, int vec_c,
                                int out_bf16, hipStream_t stream);
// The int8 / int4 weight-only head (bits 8 or 4) with bias and log-softmax;
// same stripes (q.G = lsm_workgroups(N)) and workspace as the bf16 head.
hipError_t launch_wq_thin_lsm(int bits, const W8Args& a, const LsmArgs& q, int out_bf16,
                              hipStream_t stream);
int64_t lsm_workgroups(int64_t N);
bool lsm_direct_ok(const Bf16Args& a);
hipError_t launch_quant_fp8_1x128(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quant_fp8_128x128(const QuantArgs& a, hipStream_t stream);
// Attainable-ceiling probes (measurement kernels, not part of any GEMM).
// kind 0: bf16 MFMA loop, 1: fp8 MFMA loop; one output float per thread.
int64_t probe_mfma_threads(int cus);
int64_t probe_stream_threads(int cus);
hipError_t launch_probe_mfma(int kind, int cus, int iters, uint64_t seed, float* out, hipStream_t stream);
hipError_t launch_probe_stream_read(const void* src, int64_t n16, int cus, uint32_t* out,
                                    hipStream_t stream);
const char* thin_kernel_name(int M, bool split);
const char* fp8_kernel_name(int64_t M, int64_t N, int64_t K);
bool fp8_direct_ok(int64_t M, int64_t N, int64_t K);
// The direct kernel with B as [N, K]: K % 16 == 0 and offsets below 2^31.
bool fp8_nt_ok(int64_t M, int64_t N, int64_t K);

}  // namespace tgemm
