// Small-M bf16 GEMM for gfx950, register-transposing variant: the path for
// operands the direct-to-LDS thin kernel cannot take (unaligned rows or
// strides that are not multiples of 8 elements).
//
// The LM head of the GEMM compute-cost page (section 7.2; also section 2.1,
// embedding and output layers, and section 3.2 on decode) multiplies a few
// rows X[M, K] (M = batch, often 1) by a weight W[K, N] with N in the tens
// or hundreds of thousands.  Each weight element is used M times only, so
// the kernel's job is to stream W from HBM exactly once at full bandwidth;
// the arithmetic still goes to the MFMA units (16 x 16 x 32 bf16, M padded
// up to a multiple of 16) because at M = 64 it would otherwise swamp the
// vector ALUs.
//
// Layout of the work:
//   * a workgroup owns 128 consecutive columns; its four waves split K into
//     four contiguous ranges and add their partial sums through LDS at the
//     end;
//   * per step a wave covers 32 rows of K: lane l reads 8 rows x 8 columns
//     of W (eight 16-byte loads; rows 8*(l/16) .. +7, columns 8*(l%16) .. +7)
//     and transposes them in registers.  Column c of that block becomes the
//     B operand of MFMA number c, so MFMA c computes the 16 columns
//     8*j + c (j = 0..15) and every lane ends up owning 8 consecutive output
//     columns -- W needs no trip through LDS;
//   * the loads for step s + 1 are issued before the MFMAs of step s.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 128;     // columns per workgroup
constexpr int kStepK = 32;     // K rows per wave step
constexpr int kRedStride = 132;  // floats per row of the LDS reduction buffer (padded)

// 8 bf16 of row `row`, columns col .. col+7, zero outside rows x cols,
// element by element (general instantiation).
__device__ __forceinline__ u32x4 load_row8(const uint16_t* base, int64_t ld, int row, int rows,
                                           int col, int cols) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < rows) {
    const uint16_t* p = base + static_cast<int64_t>(row) * ld + col;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col + e < cols) v[e >> 1] |= static_cast<uint32_t>(p[e]) << (16 * (e & 1));
  }
  return v;
}

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

template <int MB>
struct Stage {
  u32x4 w[8];
  u32x4 x[MB];
};

template <int MB, int EPI, bool OUT_BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void tgemm_bf16_thin(Bf16Args p) {
  apply_batch(p, OUT_BF16 ? 2 : 4);
  __shared__ float red[4 * 16 * kRedStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kCols;
  const int lc = lane & 15;   // column chunk / A row within a 16-row block
  const int kg = lane >> 4;   // 8-row K group inside a step
  const int col = n0 + 8 * lc;

  // Contiguous K range of this wave, in whole steps.
  const int steps = (p.K + kStepK - 1) / kStepK;
  const int s_begin = (steps * wave) / 4;
  const int s_end = (steps * (wave + 1)) / 4;

  f32x4 acc[MB][8];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[m][c] = f32x4{};

  // VEC: W rows k .. k+31 of this workgroup's columns, and X columns
  // k .. k+31, are read through buffer windows rebased every step; rows past
  // K or M fall outside the window and read as zero.
  const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  const uint32_t w_voff = (col < p.N) ? static_cast<uint32_t>(8 * kg * ldb2 + 16 * lc) : kOutOfRange;
  const uint32_t x_voff = static_cast<uint32_t>(lc * lda2 + 16 * kg);

  auto load = [&](Stage<MB>& st, int s) {
    const int k = s * kStepK;
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t ww = make_window(
          p.B + static_cast<int64_t>(k) * p.ldb + n0,
          (static_cast<int64_t>(p.K - k - 1) * p.ldb + (p.N - n0)) * 2);
#pragma unroll
      for (int r = 0; r < 8; ++r) st.w[r] = buf_load16(ww, w_voff, static_cast<uint32_t>(r * ldb2));
      const __amdgpu_buffer_rsrc_t wx = make_window(
          p.A + k, (static_cast<int64_t>(p.M - 1) * p.lda + (p.K - k)) * 2);
      const uint32_t xv = (k + 8 * kg < p.K) ? x_voff : kOutOfRange;
#pragma unroll
      for (int m = 0; m < MB; ++m) st.x[m] = buf_load16(wx, xv, static_cast<uint32_t>(16 * m * lda2));
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) st.w[r] = load_row8(p.B, p.ldb, k + 8 * kg + r, p.K, col, p.N);
#pragma unroll
      for (int m = 0; m < MB; ++m) st.x[m] = load_row8(p.A, p.lda, 16 * m + lc, p.M, k + 8 * kg, p.K);
    }
  };

  auto compute = [&](const Stage<MB>& st) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, transpose_col(st.w, c));
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, st.x[m]), b, acc[m][c], 0, 0, 0);
    }
  };

  Stage<MB> s0, s1;
  if (s_begin < s_end) load(s0, s_begin);
  for (int s = s_begin; s < s_end; s += 2) {
    if (s + 1 < s_end) load(s1, s + 1);
    compute(s0);
    if (s + 2 < s_end) load(s0, s + 2);
    if (s + 1 < s_end) compute(s1);
  }

  // Cross-wave reduction, one 16-row block at a time.  MFMA 16x16 accumulator
  // element i of lane l is row 4*(l/16) + i, column l%16 of its block; in
  // MFMA c that column is 8*(l%16) + c of the workgroup's 128.
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    float* mine = red + wave * 16 * kRedStride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* dst = mine + (4 * kg + i) * kRedStride + 8 * lc;
      *reinterpret_cast<f32x4*>(dst) =
          f32x4{acc[m][0][i], acc[m][1][i], acc[m][2][i], acc[m][3][i]};
      *reinterpret_cast<f32x4*>(dst + 4) =
          f32x4{acc[m][4][i], acc[m][5][i], acc[m][6][i], acc[m][7][i]};
    }
    __syncthreads();
    // Thread t finishes row t/16, columns 8*(t%16) .. +7 of this block.
    const int r = tid >> 4;
    const int cc = 8 * (tid & 15);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) s += red[(w * 16 + r) * kRedStride + cc + e];
      v[e] = s;
    }
    const int row = 16 * m + r;
    const int c0 = n0 + cc;
    if (row < p.M) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float bias = 0.0f;
        if constexpr (EPI != kEpiNone) {
          if (c0 + e < p.N) bias = bf16_bits_to_f32(p.bias[c0 + e]);
        }
        v[e] = apply_epilogue<EPI>(v[e], bias);
      }
      const int64_t off = static_cast<int64_t>(row) * p.ldc + c0;
      if constexpr (OUT_BF16) {
        uint16_t* out = static_cast<uint16_t*>(p.C) + off;
        if (c0 + 8 <= p.N && p.vec_c) {
          *reinterpret_cast<u32x4*>(out) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                 pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c0 + e < p.N) out[e] = f32_to_bf16_bits(v[e]);
        }
      } else {
        float* out = static_cast<float*>(p.C) + off;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < p.N) out[e] = v[e];
      }
    }
    __syncthreads();
  }
}

template <int MB, int EPI, bool OUT_BF16>
hipError_t launch_m(const Bf16Args& a, hipStream_t s) {
  const int grid = (a.N + kCols - 1) / kCols;
  const bool vec = a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
                   a.lda * 2 * 64 < (int64_t{1} << 31) && a.ldb * 2 * kStepK < (int64_t{1} << 31);
  if (vec) {
    hipLaunchKernelGGL((tgemm_bf16_thin<MB, EPI, OUT_BF16, true>), dim3(grid, a.batch), dim3(kThreads),
                       0, s, a);
  } else {
    hipLaunchKernelGGL((tgemm_bf16_thin<MB, EPI, OUT_BF16, false>), dim3(grid, a.batch), dim3(kThreads),
                       0, s, a);
  }
  return hipGetLastError();
}

template <int MB>
hipError_t dispatch_epi(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (out_bf16) {
    if (epi == kEpiNone) return launch_m<MB, kEpiNone, true>(a, s);
    if (epi == kEpiBias) return launch_m<MB, kEpiBias, true>(a, s);
    return launch_m<MB, kEpiBiasGelu, true>(a, s);
  }
  if (epi == kEpiNone) return launch_m<MB, kEpiNone, false>(a, s);
  if (epi == kEpiBias) return launch_m<MB, kEpiBias, false>(a, s);
  return launch_m<MB, kEpiBiasGelu, false>(a, s);
}

}  // namespace

hipError_t launch_bf16_thin_general(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (a.M <= 16) return dispatch_epi<1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_epi<2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_epi<3>(a, epi, out_bf16, s);
  return dispatch_epi<4>(a, epi, out_bf16, s);
}

}  // namespace tgemm
