// FP8 (OCP e4m3fn) GEMM with per-group fp32 scales for gfx950: the path for
// operands the direct-to-LDS kernel cannot take (rows of A or B that are not
// 16-byte multiples, such as N = 14335).
//
//   C[i, j] = sum_g sA[i, g] * sB[g, j / 128] * sum_{k in group g} A[i, k] * B[k, j]
//
// DeepGEMM page, section 2.4: low-precision inputs carry a scale per row
// group or small block (here 1 x 128 along K for A, 128 x 128 for B), the
// products are accumulated in fp32, and the scales bring the sum back to
// the output format (bf16).
//
// One K slice is exactly one scale group (BK = 128).  For every 16 x 16
// output block a wave issues one v_mfma_scale_f32_16x16x128_f8f6f4 with
// neutral block exponents (E8M0 127 = 2^0) into a zeroed temporary, which
// holds the group's exact partial sum, and then folds it into the fp32
// accumulator with a single FMA per element: acc += P_g * (sA[i, g] * sB[g, J]).
// A wave's columns lie inside one 128-column scale block of B (wave tiles
// are at most 128 wide and start on multiples of their width, which divides
// 128), so sB is one scalar per wave and slice and the row factor sA * sB is
// formed once per row.
//
// Because the accumulators are updated by vector FMAs they must live in the
// 256 architectural VGPRs (the MFMA-only AGPRs cannot be read by VALU
// instructions), so a wave owns 128 x 64 outputs (128 fp32 per lane) and a
// 256 x 128 tile is split over four waves (2 x 2), one per SIMD, which
// leaves the AGPR file free as cheap spill space.  At 4096 x 14336 that is
// 16 x 112 = 1792 tiles, exactly seven rounds of 256 compute units.  Data
// movement is the same as the bf16 tiled kernel: two LDS stages, chunk-plane
// LDS layout, and B transposed in registers (8 x 8 byte blocks) so that both
// operands are K-contiguous in LDS.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kWM = 2;  // waves along M
constexpr int kWN = 2;  // waves along N
constexpr int kThreads = 64 * kWM * kWN;
constexpr int kBM = 256;
constexpr int kBN = 128;
constexpr int kBK = 128;  // bytes of K per slice == one scale group
constexpr int kWTM = kBM / kWM;
constexpr int kWTN = kBN / kWN;
constexpr int kFM = kWTM / 16;
constexpr int kFN = kWTN / 16;
constexpr int kAStage = kBM * 8;  // 16-byte chunks
constexpr int kBStage = kBN * 8;
constexpr int kAPerThread = kAStage / kThreads;
constexpr int kRowsPerPass = kThreads / 8;  // A rows covered by one pass of the threads
constexpr int kBBlocks = (kBK / 8) * (kBN / 8);  // 8 x 8 byte blocks per B slice
constexpr int kGroupM = 4;
static_assert(128 % kWTN == 0, "a wave's columns must sit inside one 128-column scale block");
static_assert(kAStage % kThreads == 0 && kBBlocks == kThreads && kBM <= kThreads, "thread split");
static_assert(kBN / 8 * 16 == kThreads, "B mapping: 16 row groups x BN/8 column groups");
constexpr int kScaleOne = 127;    // E8M0 exponent of 1.0
constexpr int kFmtE4M3 = 0;       // f8f6f4 operand format code for FP8 E4M3

// Byte-by-byte loads of one 16-byte chunk of an A row / one 8-byte chunk of
// a B row, zero outside the matrix (general instantiation for unaligned
// rows).
__device__ __forceinline__ u32x4 load_a16_checked(const uint8_t* A, int K, int row, int M, int k) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < M) {
    const uint8_t* p = A + static_cast<int64_t>(row) * K + k;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (k + e < K) v[e >> 2] |= static_cast<uint32_t>(p[e]) << (8 * (e & 3));
  }
  return v;
}

__device__ __forceinline__ u32x2 load_b8_checked(const uint8_t* B, int N, int row, int K, int col) {
  u32x2 v = {0u, 0u};
  if (row < K) {
    const uint8_t* p = B + static_cast<int64_t>(row) * N + col;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col + e < N) v[e >> 2] |= static_cast<uint32_t>(p[e]) << (8 * (e & 3));
  }
  return v;
}

// 4 x 4 byte transpose: x[q] holds row q (bytes = columns 0..3); returns the
// four columns, each as one dword with row 0 in the low byte.
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                             uint32_t& y0, uint32_t& y1, uint32_t& y2,
                                             uint32_t& y3) {
  const uint32_t t0 = perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t t1 = perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t t2 = perm(x3, x2, 0x05010400u);
  const uint32_t t3 = perm(x3, x2, 0x07030602u);
  y0 = perm(t2, t0, 0x05040100u);
  y1 = perm(t2, t0, 0x07060302u);
  y2 = perm(t3, t1, 0x05040100u);
  y3 = perm(t3, t1, 0x07060302u);
}

template <bool VEC>
__global__ __launch_bounds__(kThreads, 1) void tgemm_fp8_bs_256x128x128(Fp8Args p, int tiles_m,
                                                                    int tiles_n) {
  __shared__ u32x4 smem[2 * (kAStage + kBStage)];
  __shared__ __attribute__((aligned(16))) float s_scale_a[2][kBM];
  u32x4* sA = smem;                 // [2][8 chunks][BM]
  u32x4* sB = smem + 2 * kAStage;   // [2][8 chunks][BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / kWN;
  const int wn = wave % kWN;

  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  const int hb = (n0 + wn * kWTN) / 128;  // this wave's B-scale column

  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{};

  // A: thread owns chunk a_c of rows a_r + 32 i.  B: thread (b_k8, b_nb) owns
  // K rows 8 b_k8 .. +7 and columns 8 b_nb .. +7; transposed, they fill half
  // (b_k8 & 1) of chunk b_k8 / 2 of eight LDS columns.
  const int a_c = tid & 7;
  const int a_r = tid >> 3;
  const int b_k8 = tid & 15;
  const int b_nb = tid >> 4;  // 0 .. BN/8 - 1
  const uint32_t a_voff = static_cast<uint32_t>(a_r * p.K + 16 * a_c);
  const uint32_t b_voff =
      (n0 + 8 * b_nb < p.N) ? static_cast<uint32_t>(8 * b_k8 * p.N + 8 * b_nb) : kOutOfRange;

  u32x4 ra[kAPerThread];
  u32x2 rb[8];
  float rs = 0.0f;

  auto gload = [&](int g) {
    const int k0 = g * kBK;
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t wa = make_window(
          p.A + static_cast<int64_t>(m0) * p.K + k0,
          static_cast<int64_t>(p.M - m0 - 1) * p.K + (p.K - k0));
      const uint32_t av = (k0 + 16 * a_c < p.K) ? a_voff : kOutOfRange;
#pragma unroll
      for (int i = 0; i < kAPerThread; ++i)
        ra[i] = buf_load16(wa, av, static_cast<uint32_t>(kRowsPerPass * i * p.K));
      const __amdgpu_buffer_rsrc_t wb = make_window(
          p.B + static_cast<int64_t>(k0) * p.N + n0,
          static_cast<int64_t>(p.K - k0 - 1) * p.N + (p.N - n0));
#pragma unroll
      for (int r = 0; r < 8; ++r) rb[r] = buf_load8(wb, b_voff, static_cast<uint32_t>(r * p.N));
    } else {
#pragma unroll
      for (int i = 0; i < kAPerThread; ++i)
        ra[i] = load_a16_checked(p.A, p.K, m0 + a_r + kRowsPerPass * i, p.M, k0 + 16 * a_c);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        rb[r] = load_b8_checked(p.B, p.N, k0 + 8 * b_k8 + r, p.K, n0 + 8 * b_nb);
    }
    if (tid < kBM) {
      const int row = m0 + tid;
      rs = row < p.M ? p.sA[static_cast<int64_t>(row) * p.G + g] : 0.0f;
    }
  };

  auto sstore = [&](int stage) {
    u32x4* a = sA + stage * kAStage + a_c * kBM + (a_r ^ a_c);
#pragma unroll
    for (int i = 0; i < kAPerThread; ++i) a[kRowsPerPass * i] = ra[i];
    if (tid < kBM) s_scale_a[stage][tid] = rs;
    // Column j of the 8 x 8 byte block gets its 8 K-bytes, rows 0..3 in the
    // low dword and rows 4..7 in the high dword.
    uint32_t col[8][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t y0, y1, y2, y3;
        transpose4x4(rb[4 * h][d], rb[4 * h + 1][d], rb[4 * h + 2][d], rb[4 * h + 3][d], y0, y1,
                     y2, y3);
        col[4 * d + 0][h] = y0;
        col[4 * d + 1][h] = y1;
        col[4 * d + 2][h] = y2;
        col[4 * d + 3][h] = y3;
      }
    }
    const int chunk = b_k8 >> 1;
    u32x2* b = reinterpret_cast<u32x2*>(sB + stage * kBStage + chunk * kBN + 8 * b_nb) + (b_k8 & 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) b[2 * (j ^ chunk)] = u32x2{col[j][0], col[j][1]};
  };

  const int lrow = lane & 15;
  const int c = 2 * (lane >> 4);  // this lane's two 16-byte chunks of the 128-byte K slice
  auto compute = [&](int stage, int g) {
    const float sb = hb < p.H ? p.sB[static_cast<int64_t>(g) * p.H + hb] : 0.0f;
    const u32x4* a_lo = sA + stage * kAStage + c * kBM + ((wm * kWTM + lrow) ^ c);
    const u32x4* a_hi = sA + stage * kAStage + (c + 1) * kBM + ((wm * kWTM + lrow) ^ (c + 1));
    const u32x4* b_lo = sB + stage * kBStage + c * kBN + ((wn * kWTN + lrow) ^ c);
    const u32x4* b_hi = sB + stage * kBStage + (c + 1) * kBN + ((wn * kWTN + lrow) ^ (c + 1));
    i32x8 fb[kFN];
#pragma unroll
    for (int j = 0; j < kFN; ++j) {  // B operands stay in registers for the slice
      const u32x4 lo = b_lo[16 * j];
      const u32x4 hi = b_hi[16 * j];
      fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const u32x4 lo = a_lo[16 * i];
      const u32x4 hi = a_hi[16 * i];
      const i32x8 fa = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      // Rows of this lane in block i: 4*(lane/16) + e.
      const f32x4 sa = *reinterpret_cast<const f32x4*>(
          &s_scale_a[stage][wm * kWTM + 16 * i + 4 * (lane >> 4)]);
      const f32x4 s = sa * sb;
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fa, fb[j], f32x4{}, kFmtE4M3, kFmtE4M3, 0, kScaleOne, 0, kScaleOne);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(part[e], s[e], acc[i][j][e]);
      }
    }
  };

  const int G = p.G;
  if (G > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    if (g + 1 < G) gload(g + 1);
    compute(g & 1, g);
    if (g + 1 < G) sstore((g + 1) & 1);
    __syncthreads();
  }

  // Epilogue: MFMA 16x16 accumulator element e of lane l is row 4*(l/16)+e,
  // column l%16 of its block.
  const int row_off = 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int col = n0 + wn * kWTN + 16 * j + lrow;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * kWTM + 16 * i + row_off + e;
        if (row < p.M && col < p.N)
          p.C[static_cast<int64_t>(row) * p.N + col] = f32_to_bf16_bits(acc[i][j][e]);
      }
    }
  }
}

}  // namespace

hipError_t launch_fp8_general(const Fp8Args& a, hipStream_t s) {
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles_n = (a.N + kBN - 1) / kBN;
  const bool vec = a.vec_a && a.vec_b && static_cast<int64_t>(a.K) * kBM < (int64_t{1} << 31) &&
                   static_cast<int64_t>(a.N) * kBK < (int64_t{1} << 31);
  if (vec) {
    hipLaunchKernelGGL(tgemm_fp8_bs_256x128x128<true>, dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                       s, a, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL(tgemm_fp8_bs_256x128x128<false>, dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                       s, a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace tgemm
