// Small-M bf16 GEMM for gfx950, written as a bandwidth-bound kernel.
//
// The LM head of the GEMM compute-cost page (section 7.2; also section 2.1,
// embedding and output layers, and section 3.2 on decode) multiplies a few
// rows X[M, K] (M = batch, often 1) by a weight W[K, N] with N in the tens
// or hundreds of thousands.  Each weight element is used M times only, so the
// kernel's job is to stream W from HBM exactly once at full bandwidth; the
// arithmetic still goes to the MFMA units (16 x 16 x 32 bf16, M padded to a
// multiple of 16) because at M = 64 it would otherwise swamp the vector ALUs.
//
// Layout of the work:
//   * a workgroup owns 512 consecutive columns, so every row of its W stripe
//     is one contiguous KiB; measured on MI355X, KiB-wide row stripes read
//     at about 6.4 TB/s against about 6.0 TB/s for 256-byte stripes;
//   * the stripe is walked in slices of 32 rows that go global -> LDS with
//     direct buffer loads (one load instruction = one row), four LDS stages
//     deep (three slices, 96 KiB, in flight per compute unit); the matching
//     16-row blocks of X come the same way;
//   * each wave owns 128 columns over the whole of K (no cross-wave
//     reduction); its MFMA B operands are read from the N-contiguous rows
//     with ds_read_b64_tr_b16, exactly as in the tiled kernel, and the
//     16-byte chunks of each LDS row are XOR-permuted so those reads are
//     bank-conflict free.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 512;        // columns per workgroup
constexpr int kWTN = 128;       // columns per wave
constexpr int kFN = kWTN / 16;  // 16-column MFMA blocks per wave
constexpr int kBK = 32;         // K rows per slice
constexpr int kNS = 4;          // LDS stages
constexpr int kWRow = kBN * 2;  // bytes per W row of the stripe (1 KiB)
constexpr int kWStage = kBK * kWRow;
constexpr int kXStage = 4 * 1024;  // four 16-row blocks of X, 64 bytes per row
constexpr int kStage = kWStage + kXStage;
constexpr int kLoadsPerSlice = kBK / 4 + 1;  // per wave: 8 W rows and one X block
static_assert(kNS * kStage <= 160 * 1024, "LDS capacity");

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// XOR on the chunk index of W row k (even, so 32-byte pairs stay together):
// the 8 rows one transposed read touches in a half-wave land in 8 different
// 32-byte bank segments.
__device__ __forceinline__ int w_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
// XOR on the chunk index of row r of an X block (4 chunks of 16 bytes).
__device__ __forceinline__ int x_swz(int r) { return (r >> 2) & 3; }

template <int MB, int EPI, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_thin(Bf16Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNS * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kBN;

  // acc[mb][j]: 16 x 16 block, transposed by the operand swap: element e of
  // lane l is row 16*mb + l%16, column 16*j + 4*(l/16) + e of the wave's 128.
  f32x4 acc[MB][kFN];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[mb][j] = f32x4{};

  // ---- global -> LDS: wave w loads W rows 8w .. 8w+7 of a slice (lane l ->
  // physical chunk l, logical chunk l ^ w_swz(row)) and X block w (rows
  // 16w .. 16w+15, lane l -> row l/4, physical chunk l%4). ----
  const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  const int xr = lane >> 2;
  const int xc = (lane & 3) ^ x_swz(xr);
  const uint32_t x_off = static_cast<uint32_t>((16 * wave + xr) * lda2 + 16 * xc);
  auto issue_slice = [&](int t) {
    const int stage = t % kNS;
    const int k0 = t * kBK;
    const i32x4 ww = make_window_words(p.B + static_cast<int64_t>(k0) * p.ldb + n0,
                                       (static_cast<int64_t>(p.K - k0 - 1) * p.ldb + (p.N - n0)) * 2);
#pragma unroll
    for (int i = 0; i < kBK / 4; ++i) {
      const int k = 8 * wave + i;
      const int c = lane ^ w_swz(k);
      buf_load16_lds(ww, smem_base + stage * kStage + k * kWRow,
                     static_cast<uint32_t>(k * ldb2 + 16 * c) | (n0 + 8 * c < p.N ? 0u : kOutOfRange));
    }
    const i32x4 wx = make_window_words(p.A + k0, (static_cast<int64_t>(p.M - 1) * p.lda + (p.K - k0)) * 2);
    buf_load16_lds(wx, smem_base + stage * kStage + kWStage + wave * 1024,
                   x_off | (k0 + 8 * xc < p.K ? 0u : kOutOfRange));
  };

  // ---- LDS -> registers ----
  // B operand of block j (columns 16 j .. +15 of the wave): lane L = 16g +
  // 4e + q supplies K row 8g + e (+4 for the second read) and columns 4q ..
  // 4q+3 of the block; it receives 4 k of column L % 16.
  const int bg = lane >> 4, be = (lane >> 2) & 3, bq = lane & 3;
  int b_off[kFN];
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int k = 8 * bg + be;
    const int chunk = (2 * (8 * wave + j) + (bq >> 1)) ^ w_swz(k);
    b_off[j] = k * kWRow + chunk * 16 + 8 * (bq & 1);
  }
  // X operand of block mb: row l%16, K 8*(l/16) .. +7 of the slice.
  const int xrow = lane & 15;
  const int x_rd = kWStage + xrow * 64 + (((lane >> 4) ^ x_swz(xrow)) * 16);

  const int KT = (p.K + kBK - 1) / kBK;
  if (KT > 0) {
    for (int t = 0; t < kNS - 1; ++t) issue_slice(t);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kNS - 2) * kLoadsPerSlice) : "memory");
    lds_barrier();
    for (int t = 0; t < KT; ++t) {
      issue_slice(t + kNS - 1);  // into the stage slice t-1 occupied
      const uint8_t* base = smem + (t % kNS) * kStage;
      bf16x8 fb[kFN], fx[MB];
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, base + b_off[j]));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, base + b_off[j] + 4 * kWRow));
        fb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        fx[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + x_rd + mb * 1024));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fx[mb], acc[mb][j], 0, 0, 0);
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
hipError_t launch_m(const Bf16Args& a, hipStream_t s) {
  hipLaunchKernelGGL((tgemm_bf16_thin<MB, EPI, OUT_BF16>), dim3((a.N + kBN - 1) / kBN),
                     dim3(kThreads), 0, s, a);
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

const char* thin_kernel_name(int M) {
  if (M <= 16) return "tgemm_bf16_thin_m16";
  if (M <= 32) return "tgemm_bf16_thin_m32";
  if (M <= 48) return "tgemm_bf16_thin_m48";
  return "tgemm_bf16_thin_m64";
}

hipError_t launch_bf16_thin(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  // Direct loads need 16-byte aligned rows and per-lane offsets below 2^31
  // (a slice's 32 rows of W, 64 rows of X).
  const bool direct = a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
                      a.ldb * 2 * kBK < (int64_t{1} << 31) && a.lda * 2 * 64 < (int64_t{1} << 31);
  if (!direct) return launch_bf16_thin_general(a, epi, out_bf16, s);
  if (a.M <= 16) return dispatch_epi<1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_epi<2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_epi<3>(a, epi, out_bf16, s);
  return dispatch_epi<4>(a, epi, out_bf16, s);
}

}  // namespace tgemm
