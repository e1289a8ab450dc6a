// Small-M GEMM with int8 weights and per-group fp32 scales (weight-only
// quantisation) for gfx950, written as a bandwidth-bound kernel.
//
//   C[i, n] = epilogue( sum_k X[i, k] * (Q[k, n] * S[k / 128, n]) + bias[n] )
//
// The GEMM compute-cost page (section 7.2, the LM head) names keeping the
// large output projection in a low-precision integer format as the first
// remedy for its memory-bound cost: the weight W[K, N] is streamed once per
// call, so halving its bytes halves the time.  Here W is stored as int8
// codes Q with one fp32 scale per (128-row group along K, column), the
// round-to-nearest per-group scheme of the DeepGEMM page's section 2.4
// applied to integers; activations X stay bf16.
//
// Layout of the work (the bf16 thin-M kernel's, with int8 rows):
//   * a workgroup owns 512 consecutive columns: a W row of its stripe is 512
//     contiguous bytes; the stripe is walked in slices of 32 rows that go
//     global -> LDS with direct buffer loads (one load = two rows), six LDS
//     stages deep, together with the matching 16-row blocks of X and the
//     512 scales of the slice's group;
//   * eight waves (two per SIMD, so one wave's conversions overlap the
//     other's MFMAs and loads) each own 64 columns over the whole of K.  A
//     wave's MFMA operand for 16 columns comes from one ds_read_b64_tr_b8
//     (lane i receives column i of 8 consecutive rows, the 8 K values one
//     16 x 16 x 32 MFMA takes per lane); each code becomes a bf16 exactly
//     (a signed byte fits bf16's 8-bit significand: sign-extending byte to
//     fp32 conversion, then the upper half), about 1.5 instructions per
//     weight;
//   * the MFMAs of a 128-row group accumulate sum_k x * q exactly as an fp32
//     GEMM would; at the end of the group one FMA per accumulator folds it
//     in with the column's scale, acc += s * partial -- the same grouped
//     dequantisation as the FP8 path, so no weight is rounded.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kThreads = 512;
constexpr int kBN = 512;        // columns per workgroup
constexpr int kWTN = 64;        // columns per wave
constexpr int kFN = kWTN / 16;  // 16-column MFMA blocks per wave
constexpr int kBK = 32;         // K rows per slice
constexpr int kGroupK = 128;    // K rows per scale group
constexpr int kNS = 6;          // LDS stages
constexpr int kWRow = kBN;      // bytes per W row of the stripe
constexpr int kWStage = kBK * kWRow;     // 16 KiB
constexpr int kXStage = 4 * 1024;        // four 16-row blocks of X, 64 bytes per row
constexpr int kSStage = kBN * 4;         // the slice group's 512 fp32 scales
constexpr int kStage = kWStage + kXStage + kSStage;
constexpr int kLoadsPerSlice = 2 + 1 + 1;  // per wave: 4 W rows, one X block, 64 scales
static_assert(kNS * kStage <= 160 * 1024, "LDS capacity");

#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// XOR on the 16-byte chunk index of W row k: the 16 rows a transposed read
// covers per 32 lanes (8g + e, g < 2, e < 8) land in 16 different 16-byte
// bank slots of a 256-byte bank row.
__device__ __forceinline__ int w8_swz(int k) { return k & 15; }
// XOR on the chunk index of row r of an X block (4 chunks of 16 bytes).
__device__ __forceinline__ int x_swz(int r) { return (r >> 2) & 3; }

// 4-byte buffer load written straight into LDS (lane l -> lds_base + 4 l).
__device__ __forceinline__ void buf_load4_lds(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_words(window))
               : "memory", "m0");
}

// Eight int8 codes (two dwords, K order) as 8 bf16, exactly.
__device__ __forceinline__ bf16x8 codes_to_bf16(i32x2 codes) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = static_cast<float>(static_cast<int8_t>(static_cast<uint32_t>(codes[0]) >> (8 * e)));
    f[4 + e] = static_cast<float>(static_cast<int8_t>(static_cast<uint32_t>(codes[1]) >> (8 * e)));
  }
  // Upper halves of two fp32 words into one (bytes 2, 3 of a then of b).
  auto hi2 = [](float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  };
  return __builtin_bit_cast(bf16x8, u32x4{hi2(f[0], f[1]), hi2(f[2], f[3]), hi2(f[4], f[5]), hi2(f[6], f[7])});
}

template <int MB, int EPI, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void tgemm_w8_thin(W8Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kBN;

  // acc[mb][j]: 16 x 16 block, transposed by the operand swap: element e of
  // lane l is row 16*mb + l%16, column 16*j + 4*(l/16) + e of the wave's 64.
  f32x4 acc[MB][kFN];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[mb][j] = f32x4{};

  // ---- global -> LDS.  W: load i of wave w covers slice rows 4w + 2i (lanes
  // 0-31) and 4w + 2i + 1 (lanes 32-63), lane -> physical chunk lane % 32,
  // logical chunk (lane % 32) ^ w8_swz(row).  X: block w % 4 (rows
  // 16(w%4) .. +15), lane -> row l/4, physical chunk l%4 (waves 4-7 write the
  // same bytes as waves 0-3, which keeps every wave's load count equal).
  // Scales: wave w fetches columns 64w .. 64w+63 of the group. ----
  const int64_t ldx2 = p.ldx * 2;
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  uint32_t w_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = 4 * wave + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ w8_swz(k);
    w_off[i] = static_cast<uint32_t>(k * p.ldq + 16 * c) | (n0 + 16 * c < p.N ? 0u : kOutOfRange);
  }
  const int xr = lane >> 2;
  const int xc = (lane & 3) ^ x_swz(xr);
  const uint32_t x_off = static_cast<uint32_t>((16 * (wave & 3) + xr) * ldx2 + 16 * xc);
  const int G = (p.K + kGroupK - 1) / kGroupK;
  auto issue_slice = [&](int t) {
    const uint32_t stage = smem_base + static_cast<uint32_t>((t % kNS) * kStage);
    const int k0 = t * kBK;
    const i32x4 ww = make_window_words(p.Q + static_cast<int64_t>(k0) * p.ldq + n0,
                                       static_cast<int64_t>(p.K - k0 - 1) * p.ldq + (p.N - n0));
#pragma unroll
    for (int i = 0; i < 2; ++i) buf_load16_lds(ww, stage + (4 * wave + 2 * i) * kWRow, w_off[i]);
    const i32x4 wx = make_window_words(p.X + k0, (static_cast<int64_t>(p.M - 1) * p.ldx + (p.K - k0)) * 2);
    buf_load16_lds(wx, stage + kWStage + (wave & 3) * 1024, x_off | (k0 + 8 * xc < p.K ? 0u : kOutOfRange));
    const int g = k0 / kGroupK;
    const i32x4 ws = make_window_words(p.S + static_cast<int64_t>(g) * p.N + n0,
                                       g < G ? static_cast<int64_t>(p.N - n0) * 4 : 0);
    buf_load4_lds(ws, stage + kWStage + kXStage + 64 * wave * 4, static_cast<uint32_t>((64 * wave + lane) * 4));
  };

  // ---- LDS -> registers ----
  // W operand of block j (columns 16 j .. +15 of the wave): within each
  // 16-lane group g, lane 2e + h supplies bytes 8h .. 8h+7 of the block in K
  // row 8g + e and receives column (lane % 16) of rows 8g .. 8g+7.
  const int bg = lane >> 4, be = (lane >> 1) & 7, bh = lane & 1;
  int b_off[kFN];
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int k = 8 * bg + be;
    b_off[j] = k * kWRow + (((4 * wave + j) ^ w8_swz(k)) * 16) + 8 * bh;
  }
  // Scales of this lane's accumulator columns 16 j + 4 (lane / 16) .. +3.
  const int s_rd = kWStage + kXStage + (kWTN * wave + 4 * (lane >> 4)) * 4;
  // X operand of block mb: row l%16, K 8*(l/16) .. +7 of the slice.
  const int xrow = lane & 15;
  const int x_rd = kWStage + xrow * 64 + (((lane >> 4) ^ x_swz(xrow)) * 16);

  const int KT = (p.K + kBK - 1) / kBK;
  if (KT > 0) {
    f32x4 part[MB][kFN];  // sum over the current 128-row group of x * q
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < kFN; ++j) part[mb][j] = f32x4{};
    for (int t = 0; t < kNS - 1; ++t) issue_slice(t);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kNS - 2) * kLoadsPerSlice) : "memory");
    lds_barrier();
    for (int t = 0; t < KT; ++t) {
      issue_slice(t + kNS - 1);  // into the stage slice t-1 occupied
      const uint8_t* base = smem + (t % kNS) * kStage;
      bf16x8 fb[kFN], fx[MB];
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        fb[j] = codes_to_bf16(__builtin_amdgcn_ds_read_tr8_b64_v2i32(TGEMM_LDS(i32x2, base + b_off[j])));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        fx[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + x_rd + mb * 1024));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
          part[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fx[mb], part[mb][j], 0, 0, 0);
      if ((t % (kGroupK / kBK)) == kGroupK / kBK - 1 || t == KT - 1) {
        // End of a scale group: acc += s * partial, per column.
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
          const f32x4 sc = *reinterpret_cast<const f32x4*>(base + s_rd + 64 * j);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][j][e] = __builtin_fmaf(part[mb][j][e], sc[e], acc[mb][j][e]);
            part[mb][j] = f32x4{};
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kNS - 2) * kLoadsPerSlice) : "memory");
      lds_barrier();  // slice t+1 landed everywhere; slice t no longer read
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
  }

  // ---- epilogue: lane holds 4 consecutive columns of one row per block ----
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int col = n0 + kWTN * wave + 16 * j + 4 * (lane >> 4);
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (EPI != kEpiNone) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < p.N) bias[e] = bf16_bits_to_f32(p.bias[col + e]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + (lane & 15);
      if (row >= p.M) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = apply_epilogue<EPI>(acc[mb][j][e], bias[e]);
      const int64_t off = static_cast<int64_t>(row) * p.ldc + col;
      const bool full = p.vec_c && col + 4 <= p.N;
      if constexpr (OUT_BF16) {
        uint16_t* out = static_cast<uint16_t*>(p.C) + off;
        if (full) {
          *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.N) out[e] = f32_to_bf16_bits(v[e]);
        }
      } else {
        float* out = static_cast<float*>(p.C) + off;
        if (full) {
          *reinterpret_cast<f32x4*>(out) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < p.N) out[e] = v[e];
        }
      }
    }
  }
}

template <int MB, int EPI, bool OUT_BF16>
hipError_t launch_m(const W8Args& a, hipStream_t s) {
  hipLaunchKernelGGL((tgemm_w8_thin<MB, EPI, OUT_BF16>), dim3((a.N + kBN - 1) / kBN), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

template <int MB>
hipError_t dispatch_epi(const W8Args& a, int epi, int out_bf16, hipStream_t s) {
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

bool w8_supported(int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq) {
  // Whole 16-byte X chunks along K, dword-aligned W rows (no dword of Q
  // straddles a window end), per-lane offsets below 2^31 (a slice's 32 rows
  // of Q, 64 rows of X), and at most 64 rows.
  return M <= 64 && K % 8 == 0 && N % 4 == 0 && ldq % 4 == 0 &&
         ldq * kBK < (int64_t{1} << 31) && ldx * 2 * 64 < (int64_t{1} << 31);
}

const char* w8_kernel_name(int M) {
  if (M <= 16) return "tgemm_w8_thin_m16";
  if (M <= 32) return "tgemm_w8_thin_m32";
  if (M <= 48) return "tgemm_w8_thin_m48";
  return "tgemm_w8_thin_m64";
}

hipError_t launch_w8_thin(const W8Args& a, int epi, int out_bf16, hipStream_t s) {
  if (a.M <= 16) return dispatch_epi<1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_epi<2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_epi<3>(a, epi, out_bf16, s);
  return dispatch_epi<4>(a, epi, out_bf16, s);
}

}  // namespace tgemm
