// Attainable-ceiling probes for gfx950: what the matrix units and HBM
// deliver on this part with nothing else in the way.  They are measurement
// kernels, not part of any GEMM: the benchmark times them next to the GEMM
// kernels and reports each kernel's fraction of these measured ceilings
// beside its fraction of the published peaks (DeepGEMM page, section 3.4:
// report time, fraction of peak and bandwidth; section 2.2: the matrix
// units must be kept fed).
//
//   * MFMA loop: every wave of a full grid (one 512-thread workgroup per
//     compute unit, two waves per SIMD) issues back-to-back MFMAs on
//     operands held in registers -- eight A and eight B fragments of
//     seeded pseudo-random values, rotated so consecutive instructions see
//     different data (constant operands draw less power and would overstate
//     the ceiling) -- into four independent accumulators.  bf16:
//     v_mfma_f32_32x32x16_bf16 (32768 FLOP); fp8: v_mfma_scale_f32_16x16x128
//     _f8f6f4 with e4m3 operands (65536 FLOP).  Each lane writes one float
//     (the sum of its accumulators) so the loop cannot be dropped.
//   * Stream read: the buffer is taken as rows of (compute units) KiB, and
//     workgroup b (one per compute unit, four waves) reads KiB b of every
//     row, eight rows in flight per wave, with non-temporal 16-byte loads --
//     so at any moment all compute units read neighbouring KiBs of the same
//     few rows.  Measured on MI355X this pattern streams at about 7.0 TB/s,
//     against about 6.0 TB/s for a grid-stride loop over the whole buffer.
//     Bytes past the last whole row are read by a grid-stride tail.  Each
//     thread XORs what it read and writes one 32-bit word, so the result can
//     be checked against the host's XOR of the same bytes.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocksPerCu = 1;
constexpr int kStreamThreads = 256;  // four waves
constexpr int kStreamRowsInFlight = 8;

// splitmix64 finaliser: a seeded value per (thread, slot).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// A random bf16 in about [-2, 2]: sign, exponent 126..127, random mantissa.
__device__ __forceinline__ uint32_t rand_bf16_pair(uint64_t r) {
  const uint32_t lo = 0x3F00u | (static_cast<uint32_t>(r) & 0x80FFu);
  const uint32_t hi = 0x3F00u | (static_cast<uint32_t>(r >> 16) & 0x80FFu);
  return lo | (hi << 16);
}

// Random e4m3 codes with exponent field 4..11 (|x| in [1/8, 30]), no NaN.
__device__ __forceinline__ uint32_t rand_e4m3_quad(uint64_t r) {
  uint32_t v = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t byte = static_cast<uint32_t>(r >> (8 * b));
    const uint32_t e = 4u + ((byte >> 3) & 7u);
    v |= ((byte & 0x80u) | (e << 3) | (byte & 7u)) << (8 * b);
  }
  return v;
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads, 1) void tgemm_probe_mfma(float* out, int iters, uint64_t seed) {
  const uint64_t t = static_cast<uint64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  float total = 0.0f;
  if constexpr (KIND == 0) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      u32x4 ua, ub;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        ua[d] = rand_bf16_pair(mix64(seed ^ (t * 64 + f * 8 + d)));
        ub[d] = rand_bf16_pair(mix64(seed ^ (t * 64 + f * 8 + 4 + d) ^ 0x5555ull));
      }
      a[f] = __builtin_bit_cast(bf16x8, ua);
      b[f] = __builtin_bit_cast(bf16x8, ub);
    }
    f32x16 acc[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + c) & 7], b[(k + 3 * c) & 7], acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) total += acc[c][e];
  } else {
    i32x8 a[8], b[8];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        a[f][d] = static_cast<int>(rand_e4m3_quad(mix64(seed ^ (t * 128 + f * 16 + d))));
        b[f][d] = static_cast<int>(rand_e4m3_quad(mix64(seed ^ (t * 128 + f * 16 + 8 + d) ^ 0xAAAAull)));
      }
    f32x4 acc[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[(k + c) & 7], b[(k + 3 * c) & 7], acc[c],
                                                                     0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) total += acc[c][e];
  }
  out[t] = total;
}

__global__ __launch_bounds__(kStreamThreads) void tgemm_probe_stream_read(const u32x4* src, int64_t n16,
                                                                        uint32_t* out) {
  constexpr int kWaves = kStreamThreads / 64;
  constexpr int U = kStreamRowsInFlight;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row16 = static_cast<int64_t>(gridDim.x) * 64;  // 16-byte units per row
  const int64_t rows = n16 / row16;
  const u32x4* base = src + static_cast<int64_t>(blockIdx.x) * 64 + lane;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  int64_t r = wave;
  for (; r + (U - 1) * kWaves < rows; r += U * kWaves) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(base + (r + u * kWaves) * row16);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  for (; r < rows; r += kWaves) x ^= __builtin_nontemporal_load(base + r * row16);
  // Tail past the last whole row.
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kStreamThreads + threadIdx.x;
  for (int64_t i = rows * row16 + t; i < n16; i += static_cast<int64_t>(gridDim.x) * kStreamThreads)
    x ^= src[i];
  out[t] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace

int64_t probe_mfma_threads(int cus) { return static_cast<int64_t>(cus) * kProbeBlocksPerCu * kProbeThreads; }
int64_t probe_stream_threads(int cus) { return static_cast<int64_t>(cus) * kStreamThreads; }

hipError_t launch_probe_mfma(int kind, int cus, int iters, uint64_t seed, float* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(cus * kProbeBlocksPerCu));
  if (kind == 0)
    hipLaunchKernelGGL(tgemm_probe_mfma<0>, grid, dim3(kProbeThreads), 0, s, out, iters, seed);
  else
    hipLaunchKernelGGL(tgemm_probe_mfma<1>, grid, dim3(kProbeThreads), 0, s, out, iters, seed);
  return hipGetLastError();
}

hipError_t launch_probe_stream_read(const void* src, int64_t n16, int cus, uint32_t* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(cus));
  hipLaunchKernelGGL(tgemm_probe_stream_read, grid, dim3(kStreamThreads), 0, s,
                     static_cast<const u32x4*>(src), n16, out);
  return hipGetLastError();
}

}  // namespace tgemm
