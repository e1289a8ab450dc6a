// LDS-tiled bf16 GEMM for gfx950: C = epilogue(A . B + bias), fp32 accumulate.
//
// Structure (DeepGEMM page, sections 2.1-2.3 and 3.3; tensor-core page,
// "Chunking" and "Registers与Tensor Cores"):
//   * tiling -- each workgroup owns one BM x BN output tile and walks K in
//     slices of BK = 64; four waves split the tile 2 x 2, so each wave owns
//     a (BM/2) x (BN/2) block of 32 x 32 MFMA accumulators in registers;
//   * staging -- every K slice of A (BM x 64) and B (64 x BN) is fetched with
//     16-byte buffer loads into registers and written to LDS.  B arrives
//     N-contiguous and is transposed 8 x 8 in registers on the way, so both
//     operands sit K-contiguous in LDS, which is the layout the MFMA operand
//     registers take;
//   * pipelining -- two LDS stages; the global loads of slice t+1 are in
//     flight while the MFMAs of slice t run, with one barrier per slice;
//   * bank conflicts -- chunk-plane LDS layout with an XOR of the row's low
//     bits (see plane_slot);
//   * epilogue -- bias, tanh-GeLU and the output rounding are applied to the
//     fp32 accumulators before the single store (GEMM compute-cost page,
//     section 5.1); rows and columns past M, N are masked, and the K tail is
//     zero-filled on both operands (DeepGEMM page, section 4.1).
//
// Two instantiations per shape: VEC (aligned operands whose inner extents are
// multiples of 8; edges handled by out-of-range buffer offsets, which read as
// zero) and a general one that assembles edge chunks element by element.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kGroupM = 4;  // tile-rows per scheduling group

template <int BM_, int BN_>
struct Tiled {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int WTM = BM / 2;  // wave tile (2 x 2 waves)
  static constexpr int WTN = BN / 2;
  static constexpr int FM = WTM / 32;  // 32 x 32 MFMA blocks per wave
  static constexpr int FN = WTN / 32;
  static constexpr int A_PER_THREAD = BM * 8 / kThreads;  // 16-byte chunks of A per thread
  static constexpr int B_THREADS = BN;                     // threads owning an 8 x 8 B block
  static constexpr int A_STAGE = BM * 8;                   // 16-byte slots per LDS stage
  static constexpr int B_STAGE = BN * 8;
  static constexpr int LDS_SLOTS = 2 * (A_STAGE + B_STAGE);
  static_assert((BM * 8) % kThreads == 0, "A slice must split evenly over the threads");
  static_assert(BN <= kThreads, "one thread per 8 x 8 block of the B slice");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32 x 32 block");
};

// 16-byte chunk (8 bf16) of row `row`, columns col .. col+7, zero outside
// rows x cols; element by element (general instantiation).
__device__ __forceinline__ u32x4 load16_checked(const uint16_t* base, int64_t ld, int row, int rows,
                                                int col, int cols) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < rows) {
    const uint16_t* p = base + static_cast<int64_t>(row) * ld + col;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (col + e < cols) v[e >> 1] |= static_cast<uint32_t>(p[e]) << (16 * (e & 1));
    }
  }
  return v;
}

// Column j of an 8 x 8 bf16 block given as 8 rows (k) of 8 columns (n): the 8
// k-values of that column, two per dword, low half first.
__device__ __forceinline__ u32x4 transpose_col(const u32x4 (&r)[8], int j) {
  const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  const int d = j >> 1;
  u32x4 o;
  o[0] = perm(r[1][d], r[0][d], sel);
  o[1] = perm(r[3][d], r[2][d], sel);
  o[2] = perm(r[5][d], r[4][d], sel);
  o[3] = perm(r[7][d], r[6][d], sel);
  return o;
}

template <class T, int EPI, bool OUT_BF16, bool VEC>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_tiled(Bf16Args p, int tiles_m,
                                                                int tiles_n) {
  __shared__ u32x4 smem[T::LDS_SLOTS];
  u32x4* sA = smem;                   // [2][8 chunks][BM]
  u32x4* sB = smem + 2 * T::A_STAGE;  // [2][8 chunks][BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * T::BM;
  const int n0 = tn * T::BN;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x16{};

  // A: thread owns chunk a_c of rows a_r + 32 i.  B: thread (b_kb, b_nb) owns
  // K rows 8 b_kb .. +7 and columns 8 b_nb .. +7 of the slice.
  const int a_c = tid & 7;
  const int a_r = tid >> 3;
  const int b_kb = tid & 7;
  const int b_nb = tid >> 3;
  const bool b_owner = tid < T::B_THREADS;
  const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  const uint32_t a_voff = static_cast<uint32_t>(a_r * lda2 + 16 * a_c);
  const uint32_t b_voff_ok = static_cast<uint32_t>(8 * b_kb * ldb2 + 16 * b_nb);
  const uint32_t b_voff = (b_owner && n0 + 8 * b_nb < p.N) ? b_voff_ok : kOutOfRange;

  u32x4 ra[T::A_PER_THREAD];
  u32x4 rb[8];

  auto gload = [&](int k0) {
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t wa = make_window(
          p.A + static_cast<int64_t>(m0) * p.lda + k0,
          (static_cast<int64_t>(p.M - m0 - 1) * p.lda + (p.K - k0)) * 2);
      const uint32_t av = (k0 + 8 * a_c < p.K) ? a_voff : kOutOfRange;
#pragma unroll
      for (int i = 0; i < T::A_PER_THREAD; ++i)
        ra[i] = buf_load16(wa, av, static_cast<uint32_t>(32 * i * lda2));
      const __amdgpu_buffer_rsrc_t wb = make_window(
          p.B + static_cast<int64_t>(k0) * p.ldb + n0,
          (static_cast<int64_t>(p.K - k0 - 1) * p.ldb + (p.N - n0)) * 2);
      if (b_owner) {
#pragma unroll
        for (int r = 0; r < 8; ++r) rb[r] = buf_load16(wb, b_voff, static_cast<uint32_t>(r * ldb2));
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::A_PER_THREAD; ++i)
        ra[i] = load16_checked(p.A, p.lda, m0 + a_r + 32 * i, p.M, k0 + 8 * a_c, p.K);
      if (b_owner) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          rb[r] = load16_checked(p.B, p.ldb, k0 + 8 * b_kb + r, p.K, n0 + 8 * b_nb, p.N);
      }
    }
  };

  auto sstore = [&](int stage) {
    u32x4* a = sA + stage * T::A_STAGE + a_c * T::BM + (a_r ^ a_c);
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) a[32 * i] = ra[i];
    if (b_owner) {
      u32x4* b = sB + stage * T::B_STAGE + b_kb * T::BN + 8 * b_nb;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j ^ b_kb] = transpose_col(rb, j);
    }
  };

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  auto compute = [&](int stage) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = 2 * ks + lhalf;
      const u32x4* a = sA + stage * T::A_STAGE + c * T::BM + ((wm * T::WTM + lrow) ^ c);
      const u32x4* b = sB + stage * T::B_STAGE + c * T::BN + ((wn * T::WTN + lrow) ^ c);
      bf16x8 fa[T::FM], fb[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i) fa[i] = __builtin_bit_cast(bf16x8, a[32 * i]);
#pragma unroll
      for (int j = 0; j < T::FN; ++j) fb[j] = __builtin_bit_cast(bf16x8, b[32 * j]);
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  const int KT = (p.K + kBK - 1) / kBK;
  if (KT > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int t = 0; t < KT; ++t) {
    if (t + 1 < KT) gload((t + 1) * kBK);
    compute(t & 1);
    if (t + 1 < KT) sstore((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: MFMA 32x32 accumulator element 4*g + e of lane l is row
  // 8*g + 4*(l/32) + e, column l%32 of its block.
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int col = n0 + wn * T::WTN + 32 * j + lrow;
    float bias = 0.0f;
    if constexpr (EPI != kEpiNone) {
      if (col < p.N) bias = bf16_bits_to_f32(p.bias[col]);
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int rbase = m0 + wm * T::WTM + 32 * i + 4 * lhalf;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + 8 * g + e;
          if (row < p.M && col < p.N) {
            const float v = apply_epilogue<EPI>(acc[i][j][4 * g + e], bias);
            const int64_t off = static_cast<int64_t>(row) * p.ldc + col;
            if constexpr (OUT_BF16) {
              static_cast<uint16_t*>(p.C)[off] = f32_to_bf16_bits(v);
            } else {
              static_cast<float*>(p.C)[off] = v;
            }
          }
        }
      }
    }
  }
}

template <class T, int EPI, bool OUT_BF16>
hipError_t launch_t(const Bf16Args& a, hipStream_t s) {
  const int tiles_m = (a.M + T::BM - 1) / T::BM;
  const int tiles_n = (a.N + T::BN - 1) / T::BN;
  const int total = tiles_m * tiles_n;
  const bool vec = a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
                   a.lda * 2 * T::BM < (int64_t{1} << 31) && a.ldb * 2 * kBK < (int64_t{1} << 31);
  if (vec) {
    hipLaunchKernelGGL((tgemm_bf16_tiled<T, EPI, OUT_BF16, true>), dim3(total), dim3(kThreads), 0,
                       s, a, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((tgemm_bf16_tiled<T, EPI, OUT_BF16, false>), dim3(total), dim3(kThreads), 0,
                       s, a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_epi(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (out_bf16) {
    if (epi == kEpiNone) return launch_t<T, kEpiNone, true>(a, s);
    if (epi == kEpiBias) return launch_t<T, kEpiBias, true>(a, s);
    return launch_t<T, kEpiBiasGelu, true>(a, s);
  }
  if (epi == kEpiNone) return launch_t<T, kEpiNone, false>(a, s);
  if (epi == kEpiBias) return launch_t<T, kEpiBias, false>(a, s);
  return launch_t<T, kEpiBiasGelu, false>(a, s);
}

}  // namespace

TiledShapeInfo tiled_shape_info(int shape) {
  switch (shape) {
    case kTile256x256: return {256, 256, "tgemm_bf16_tiled_256x256x64"};
    case kTile256x128: return {256, 128, "tgemm_bf16_tiled_256x128x64"};
    default: return {128, 128, "tgemm_bf16_tiled_128x128x64"};
  }
}

hipError_t launch_bf16_tiled(const Bf16Args& a, int shape, int epi, int out_bf16,
                             hipStream_t s) {
  switch (shape) {
    case kTile256x256: return dispatch_epi<Tiled<256, 256>>(a, epi, out_bf16, s);
    case kTile256x128: return dispatch_epi<Tiled<256, 128>>(a, epi, out_bf16, s);
    default: return dispatch_epi<Tiled<128, 128>>(a, epi, out_bf16, s);
  }
}

}  // namespace tgemm
