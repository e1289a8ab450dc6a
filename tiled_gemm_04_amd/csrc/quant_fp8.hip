// FP8 (OCP e4m3fn) quantisers with per-group fp32 scales for gfx950: the
// producers of gemm_fp8_blockscaled's operands.
//
// DeepGEMM page, section 2.4: a row group or a small block of values shares
// one scale that maps it into the narrow FP8 range; the groups here are the
// ones the block-scaled GEMM consumes -- (row, 128 consecutive columns) of
// the activation matrix and 128 x 128 blocks of the weight matrix.  Per
// group, in fp32:
//
//   amax  = max |x| over the group's elements inside the matrix
//   scale = amax / 448 (rounded to nearest), or 1 when amax == 0
//   code  = e4m3( clamp(x / scale, -448, 448) ), x / scale rounded to
//           nearest, the e4m3 cast to nearest with ties to even
//
// Every code is the integer a plain fp32 evaluation of those formulas gives:
// the quotient is the correctly rounded one (see quotient) and the cast
// rounds to nearest even.
//
// Mapping onto CDNA4: both are single-pass, HBM-bound kernels.  The 1 x 128
// kernel works in tasks of 512 consecutive columns of one row (four groups):
// a lane holds 8 values (one 16-byte load), the 16 lanes of a group reduce
// their maxima with cross-lane shuffles, and each lane writes its 8 codes
// (8 bytes) -- a task reads 1 KiB and writes 512 bytes, contiguous.  One
// task per wave measured fastest (more waves in flight than batching several
// tasks' loads in one wave).  The
// 128 x 128 kernel gives each 256-thread workgroup one block: every thread
// keeps its 64 values in registers while the block maximum is formed (wave
// shuffles, then four partial maxima through LDS), so the block is read from
// HBM once.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kGroup = 128;
using fp8q::codes8;
using fp8q::group_scale;

// Eight bf16 values of one row starting at column c (columns >= ncols read
// as 0; a zero never changes a group maximum).
__device__ __forceinline__ void load8(const uint16_t* row, int64_t c, int64_t ncols, bool vec, float (&v)[8]) {
  if (vec && c + 8 <= ncols) {
    const u32x4 d = *reinterpret_cast<const u32x4*>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(d[e] << 16);
      v[2 * e + 1] = __uint_as_float(d[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = c + e < ncols ? bf16_bits_to_f32(row[c + e]) : 0.0f;
  }
}

// Eight codes of one row starting at column c (columns >= ncols skipped).
// The codes are written once and not read back by this kernel: whole 8-byte
// stores carry the non-temporal hint (measured 4 % faster on the 1 x 128
// quantiser and 12 % on the 128 x 128 one; the same hint on the loads made
// both slower).
__device__ __forceinline__ void store8(uint8_t* row, int64_t c, int64_t ncols, bool vec, u32x2 q) {
  if (vec && c + 8 <= ncols) {
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(row + c));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < ncols) row[c + e] = static_cast<uint8_t>(q[e / 4] >> (8 * (e % 4)));
  }
}

// ---- 1 x 128 groups: each wave takes kTasks consecutive (row, 512-column)
// tasks of the row-major task list, loads first ----
constexpr int kTasks = 1;

__global__ __launch_bounds__(256) void tgemm_quant_fp8_1x128(QuantArgs p, int64_t tasks) {
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (p.cols + 511) / 512;
  float v[kTasks][8];
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int64_t task = w * kTasks + k;
    const int64_t r = task / chunks;
    const int64_t c = (task % chunks) * 512 + 8 * lane;
    if (task < tasks) {
      load8(p.X + r * p.ldx, c, p.cols, p.vec_in, v[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] = 0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int64_t task = w * kTasks + k;
    if (task >= tasks) break;  // wave-uniform
    const int64_t r = task / chunks;
    const int64_t c = (task % chunks) * 512 + 8 * lane;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[k][e]));
    // Lanes 16q .. 16q+15 hold group q of the task's 512 columns.
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, d, 64));
    const float scale = group_scale(amax);
    store8(p.Q + r * p.cols, c, p.cols, p.vec_out, codes8(v[k], scale));
    if ((lane & 15) == 0 && c < p.cols) p.S[r * p.groups_per_row + c / kGroup] = scale;
  }
}

// ---- 128 x 128 blocks: one 256-thread workgroup per block ----
// Thread t handles the 16-byte chunks t + 256 j (j < 8) of the block: chunk
// i is row i / 16, columns 8 (i % 16) .. +7 of the block, so a wave reads
// four 256-byte row segments per load.
__global__ __launch_bounds__(256) void tgemm_quant_fp8_128x128(QuantArgs p, int blocks_per_row) {
  __shared__ float part[4];
  const int t = threadIdx.x;
  const int64_t bg = blockIdx.x / blocks_per_row;  // block row
  const int64_t bh = blockIdx.x % blocks_per_row;  // block column
  const int64_t r0 = bg * kGroup, c0 = bh * kGroup;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = t + 256 * j;
    const int64_t r = r0 + i / 16;
    const int64_t c = c0 + 8 * (i % 16);
    if (r < p.rows) {
      load8(p.X + r * p.ldx, c, p.cols, p.vec_in, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j][e]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, d, 64));
  if ((t & 63) == 0) part[t >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(part[0], part[1]), __builtin_fmaxf(part[2], part[3]));
  const float scale = group_scale(amax);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = t + 256 * j;
    const int64_t r = r0 + i / 16;
    const int64_t c = c0 + 8 * (i % 16);
    if (r < p.rows) store8(p.Q + r * p.cols, c, p.cols, p.vec_out, codes8(v[j], scale));
  }
  if (t == 0) p.S[bg * p.groups_per_row + bh] = scale;
}

}  // namespace

hipError_t launch_quant_fp8_1x128(const QuantArgs& a, hipStream_t s) {
  const int64_t tasks = a.rows * ((a.cols + 511) / 512);
  const int64_t waves = (tasks + kTasks - 1) / kTasks;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(tgemm_quant_fp8_1x128, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, tasks);
  return hipGetLastError();
}

hipError_t launch_quant_fp8_128x128(const QuantArgs& a, hipStream_t s) {
  const int64_t br = (a.rows + kGroup - 1) / kGroup, bc = (a.cols + kGroup - 1) / kGroup;
  if (br * bc > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(tgemm_quant_fp8_128x128, dim3(static_cast<unsigned>(br * bc)), dim3(256), 0, s, a,
                     static_cast<int>(bc));
  return hipGetLastError();
}

}  // namespace tgemm
