// Device-side helpers shared by the gfx950 GEMM kernels.
//
// Everything here is written for CDNA4 (gfx950, wave64, MFMA matrix cores,
// 160 KB of LDS per compute unit).  Sources cited by short name:
// "DeepGEMM page" = zwxr.cn/news/240083, "GEMM compute-cost page" =
// kwkr.cn/news/191298, "tensor-core page" = llmtrend.com, 大语言模型（LLM）
// 推理加速的秘诀：矩阵乘法、tensor-core.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tgemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte vectors at 2- or 4-byte alignment: stored with one 16-byte global
// store (the memory path on gfx950 takes any byte address), for output rows
// that are not 16-byte aligned.
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator dies, 32 CUs each

enum Epilogue { kEpiNone = 0, kEpiBias = 1, kEpiBiasGelu = 2 };

// ---------------------------------------------------------------- bf16 ---

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16; the hardware conversion
// (v_cvt_pk_bf16_f32) is what a plain __bf16 cast lowers to on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two values in one v_cvt_pk_bf16_f32 (lo in bits 15:0).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// -------------------------------------------------------------- epilogue ---

// tanh-form GeLU.  0.5*(1 + tanh(u)) equals the logistic function at 2u, so
// gelu(y) = y / (1 + exp(-2u)) with u = sqrt(2/pi) * (y + 0.044715 y^3); this
// form has no cancellation for large negative y (exp overflows to +inf and
// the reciprocal to 0).  exp is taken as 2^x with the hardware v_exp_f32 and
// the division as a product with v_rcp_f32 (both about 1 ulp, far below
// the bf16 output's rounding).
__device__ __forceinline__ float gelu_tanh(float y) {
  constexpr float kSqrt2OverPi = 0.7978845608028654f;
  constexpr float kCubic = 0.044715f;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kA = -2.0f * kLog2e * kSqrt2OverPi;  // exponent = y * (kA + kB y^2)
  constexpr float kB = kA * kCubic;
  const float e = __builtin_amdgcn_exp2f(y * __builtin_fmaf(kB, y * y, kA));
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int EPI>
__device__ __forceinline__ float apply_epilogue(float acc, float bias) {
  if constexpr (EPI == kEpiNone) {
    return acc;
  } else if constexpr (EPI == kEpiBias) {
    return acc + bias;
  } else {
    return gelu_tanh(acc + bias);
  }
}

// --------------------------------------------------- FP8 quantisation ---

// Per-group FP8 (OCP e4m3fn) quantisation of fp32 values, shared by the
// standalone quantisers and the bf16 GEMM's quantising epilogue so both give
// the same codes for the same inputs (DeepGEMM page, section 2.4: a group of
// values shares one fp32 scale that maps it into the e4m3 range):
//   scale = amax / 448 (1 when amax == 0), code = e4m3(clamp(x / scale)).
namespace fp8q {

constexpr float kE4m3Max = 448.0f;  // largest finite e4m3fn value

__device__ __forceinline__ float group_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4m3Max;
}

// x / scale rounded to nearest in fp32, from inv = 1/scale rounded to
// nearest (one correctly rounded division per group): q0 = x * inv, then
// one correction with the exact remainder x - scale * q0 (an FMA).  With inv
// correctly rounded and q0 within one ulp, q0 + remainder * inv rounded is
// the correctly rounded quotient (Markstein's division step); checked equal
// to the IEEE division on 4 million random operand pairs of this form on
// MI355X.  A zero quotient takes x's sign, as the division gives -0 for -0.
__device__ __forceinline__ float quotient(float x, float scale, float inv) {
  const float q0 = x * inv;
  const float q = __builtin_fmaf(__builtin_fmaf(-scale, q0, x), inv, q0);
  return __builtin_copysignf(q, x);
}

// e4m3fn codes of two values already clamped to [-448, 448], to nearest
// with ties to even (v_cvt_pk_fp8_f32; its codes for every bf16 value, every
// rounding tie and 8 million random fp32 values in that range equal a
// bit-level rounding of the 23-bit mantissa to 3 bits, subnormals included),
// in the low 16 bits of the result.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// Eight codes of x[0..7] under one group scale, packed little-endian.
__device__ __forceinline__ u32x2 codes8(const float (&x)[8], float scale) {
  const float inv = 1.0f / scale;
  float c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c[e] = __builtin_amdgcn_fmed3f(quotient(x[e], scale, inv), -kE4m3Max, kE4m3Max);
  return u32x2{e4m3_pair(c[0], c[1]) | (e4m3_pair(c[2], c[3]) << 16),
               e4m3_pair(c[4], c[5]) | (e4m3_pair(c[6], c[7]) << 16)};
}

}  // namespace fp8q

// ----------------------------------------------------------- scheduling ---

// Workgroups are dealt round-robin to the 8 dies (workgroup w runs on die
// w % 8), and each die has its own L2.  Renumber so that each die receives a
// contiguous run of logical tile ids; neighbouring logical tiles share rows
// of A or columns of B and so hit the same L2.  Bijective on [0, total).
__device__ __forceinline__ int xcd_remap(int w, int total) {
  int per = total / kNumXcd;
  int rem = total % kNumXcd;
  int xcd = w % kNumXcd;
  int idx = w / kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Grouped ordering of a tiles_m x tiles_n grid: runs of `group` tile-rows are
// walked column by column, so consecutive logical ids form compact blocks.
__device__ __forceinline__ void tile_coords(int logical, int tiles_m, int tiles_n, int group,
                                            int& tm, int& tn) {
  int per_group = group * tiles_n;
  int gid = logical / per_group;
  int first_m = gid * group;
  int gsize = tiles_m - first_m < group ? tiles_m - first_m : group;
  int in_group = logical - gid * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// ------------------------------------------------------------------- LDS ---

// Operand tiles live in LDS as "chunk planes": for a tile of R rows whose
// K extent is 8 chunks of 16 bytes, chunk c of row r sits at 16-byte slot
//   c * R + (r ^ c)            (c < 8, so the XOR only permutes r's low 3 bits).
// Eight lanes that read one chunk of eight consecutive rows, or write eight
// different chunks of one row, always hit eight different 16-byte bank groups;
// and because the XOR never touches bits 3 and up, rows 16 or 32 apart keep a
// constant slot distance, so every MFMA block of a wave is addressed from a
// single base register with immediate offsets.
__device__ __forceinline__ int plane_slot(int rows, int r, int c) { return c * rows + (r ^ c); }

// ------------------------------------------------------------- buffers ---

// Buffer resource over [base, base + bytes), bytes clamped to 2^31 - 1.
// Raw buffer loads whose offset falls outside the range return zero instead
// of touching memory; the kernels use that for the edge rows of a tile and
// pass kOutOfRange as the offset of any chunk that lies past M, N or K.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kBufferFlags = 0x00020000u;  // dword 3: 32-bit data format, no swizzle

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_window(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           static_cast<int>(kBufferFlags));
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// The same window as a plain 4-dword descriptor, for inline assembly.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_window_words(const void* base, int64_t bytes) {
  // Clamp to [0, 2^31 - 1] with 32-bit compares only (the scalar unit has no
  // 64-bit signed compare; a vector compare would move the descriptor into
  // vector registers).
  const uint64_t u = static_cast<uint64_t>(bytes);
  const int32_t hi = static_cast<int32_t>(u >> 32);
  const uint32_t lo = static_cast<uint32_t>(u);
  const int32_t n = hi < 0 ? 0 : ((hi > 0 || lo > 0x7fffffffu) ? 0x7fffffff : static_cast<int32_t>(lo));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int32_t>(a & 0xffffffffu), static_cast<int32_t>((a >> 32) & 0xffffu), n,
               static_cast<int32_t>(kBufferFlags)};
}

// 16-byte buffer load written straight into LDS: lane l's 16 bytes land at
// LDS byte address lds_base + 16 l (lds_base must be wave-uniform), offsets
// outside the window write zeros.  Emitted as inline assembly so the compiler
// does not guard every later LDS read with a wait for all outstanding loads;
// callers order these loads themselves with vmcnt waits and barriers.
// The descriptor and base must be wave-uniform; readfirstlane makes that
// explicit to the compiler (and costs nothing for values already scalar).
__device__ __forceinline__ i32x4 uniform_words(i32x4 w) {
  return i32x4{__builtin_amdgcn_readfirstlane(w[0]), __builtin_amdgcn_readfirstlane(w[1]),
               __builtin_amdgcn_readfirstlane(w[2]), __builtin_amdgcn_readfirstlane(w[3])};
}
__device__ __forceinline__ void buf_load16_lds(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_words(window))
               : "memory", "m0");
}
// The same load for a descriptor already made uniform (uniform_words, once,
// before a loop), passed to the instruction as scalar registers as it is.  A
// readfirstlane per load makes the compiler keep a loop-invariant descriptor
// in vector registers and copy it back for every load.
__device__ __forceinline__ void buf_load16_lds_u(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(window)
               : "memory", "m0");
}

__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// ------------------------------------------------------------ byte moves ---

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value
// (hi:lo).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ------------------------------------------------------------ scheduling ---

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its
// outstanding global loads (those are the prefetch of a later slice).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

#define TGEMM_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Slot of item k when n items are spread evenly over slots [a, b).
__host__ __device__ constexpr int spread(int k, int n, int a, int b) { return a + (k * (b - a)) / n; }

// f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N-1>),
// expanded at compile time so every index is a constant.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace tgemm
