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
//   * the stripe is walked in slices of 32 rows (one 16-byte load
//     instruction per wave = one KiB row), with the matching 16-row blocks of
//     X, in one of two pipelines:
//       - register-staged (grids of at least three quarters of the
//         compute units): each wave keeps two slices in flight in
//         registers, loaded with the non-temporal hint, and writes each to
//         one of two LDS stages before it is used.  At any moment every
//         compute unit reads neighbouring KiBs of the same few W rows, the
//         pattern that streams fastest on MI355X (about 7.0 TB/s, against
//         about 6.3 TB/s for the same rows through direct loads into LDS,
//         which take no cache hint);
//       - direct-to-LDS (smaller grids and the split-K kernel, where each
//         unit's rate is bounded by the bytes it keeps in flight): buffer
//         loads write LDS themselves, four stages deep (three slices,
//         96 KiB, in flight per compute unit);
//   * each wave owns 128 columns over the whole of K (no cross-wave
//     reduction); its MFMA B operands are read from the N-contiguous rows
//     with ds_read_b64_tr_b16, exactly as in the tiled kernel, and the
//     16-byte chunks of each LDS row are XOR-permuted so those reads are
//     bank-conflict free.
#include "common.h"
#include "launch.h"

#include <mutex>

// Device scratch of the allocation-free split entry point (gemm_bf16_noalloc):
// the fp32 partials of the small-M K split, in a fixed array that every GPU
// the library runs on holds for the life of the process.  Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol): it takes each device's address of the array from
// hipGetSymbolAddress (noalloc_scratch below) and passes that to the kernels.
static __device__ __align__(256) float scratch[tgemm::kNoAllocScratchBytes / sizeof(float)];

namespace tgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 512;        // columns per workgroup
constexpr int kWTN = 128;       // columns per wave
constexpr int kFN = kWTN / 16;  // 16-column MFMA blocks per wave
constexpr int kBK = 32;         // K rows per slice
constexpr int kNSReg = 2;       // LDS stages, register-staged pipeline
constexpr int kNSLds = 4;       // LDS stages, direct-to-LDS pipeline
constexpr int kWRow = kBN * 2;  // bytes per W row of the stripe (1 KiB)
constexpr int kWStage = kBK * kWRow;
constexpr int kXStage = 4 * 1024;  // four 16-row blocks of X, 64 bytes per row
constexpr int kStage = kWStage + kXStage;
constexpr int kWRows = kBK / 4;  // W rows per wave and slice
constexpr int kLoadsPerSlice = kWRows + 1;  // direct-to-LDS loads per wave and slice
constexpr uint32_t kCacheNT = 2;  // buffer-load cache policy: non-temporal
static_assert(kNSLds * kStage <= 160 * 1024, "LDS capacity");

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// XOR on the chunk index of W row k (even, so 32-byte pairs stay together):
// the 8 rows one transposed read touches in a half-wave land in 8 different
// 32-byte bank segments.
__device__ __forceinline__ int w_swz(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }
// XOR on the chunk index of row r of an X block (4 chunks of 16 bytes).
__device__ __forceinline__ int x_swz(int r) { return (r >> 2) & 3; }

// One slice of one wave in flight: its 8 W rows and its X block, 16 bytes
// per lane each.
struct SliceRegs {
  u32x4 w[kWRows];
  u32x4 x;
};

// Buffer descriptor over [base, base + bytes), bytes clamped to [0, 2^31 - 1]
// with 32-bit compares so the descriptor stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window32(const void* base, int64_t bytes) {
  const uint64_t u = static_cast<uint64_t>(bytes);
  const int32_t hi = static_cast<int32_t>(u >> 32);
  const uint32_t lo = static_cast<uint32_t>(u);
  const int32_t n = hi < 0 ? 0 : ((hi > 0 || lo > 0x7fffffffu) ? 0x7fffffff : static_cast<int32_t>(lo));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           static_cast<int>(kBufferFlags));
}

// The register-staged pipeline streams fastest when the grid covers the
// chip; with fewer workgroups each compute unit's share of the stream is
// bounded by the bytes it keeps in flight, and the deeper direct-to-LDS
// pipeline wins.  Register staging from three quarters of the compute units.
bool use_reg_pipeline(int64_t workgroups) { return 4 * workgroups >= 3 * static_cast<int64_t>(device_cus()); }

// Streams the workgroup's 512-column stripe of W once and leaves the
// products in acc[mb][j] (16 x 16 blocks, transposed by the operand swap:
// element e of lane l is row 16*mb + l%16, column 16*j + 4*(l/16) + e of the
// wave's 128).  Slices [tb, te) of K (te < 0: through the last) are summed;
// the end of the range acts as K, so nothing past it is loaded.  REG picks
// the register-staged pipeline (two LDS stages) over the direct-to-LDS one
// (four stages); smem must hold that many.  Ends with no load still writing
// LDS; the caller synchronises the workgroup before reusing smem.
template <int MB, bool REG>
__device__ __forceinline__ void thin_accumulate(const Bf16Args& p, uint8_t* smem, f32x4 (&acc)[MB][kFN],
                                                int tb = 0, int te = -1) {
  constexpr int NS = REG ? kNSReg : kNSLds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kBN;

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[mb][j] = f32x4{};

  // ---- global -> LDS (through registers or directly): wave w loads W
  // rows 8w .. 8w+7 of a slice (lane l reads logical chunk l ^ w_swz(row)
  // and stores it as physical chunk l) and X block w (rows 16w .. 16w+15,
  // lane l -> row l/4, physical chunk l%4).  Each lane's offsets within a
  // slice do not depend on the slice; columns past N are flagged out of
  // range (read as zero). ----
  const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  uint32_t w_off[kWRows];
#pragma unroll
  for (int i = 0; i < kWRows; ++i) {
    const int k = kWRows * wave + i;
    const int c = lane ^ w_swz(k);
    w_off[i] = static_cast<uint32_t>(k * ldb2 + 16 * c) | (n0 + 8 * c < p.N ? 0u : kOutOfRange);
  }
  const int xr = lane >> 2;
  const int xc = (lane & 3) ^ x_swz(xr);
  const uint32_t x_off = static_cast<uint32_t>((16 * wave + xr) * lda2 + 16 * xc);
  const int KT = (p.K + kBK - 1) / kBK;
  if (te < 0) te = KT;
  const int kend = p.K < te * kBK ? p.K : te * kBK;  // this range's end of K
  // Slice t into registers.  W rows are read once by the whole grid and go
  // with the non-temporal hint; the X block is re-read by every workgroup
  // and stays cacheable.  Slices at or past the range's end get empty
  // windows: their loads read nothing and return zeros.
  auto load_slice = [&](int t, SliceRegs& r) {
    const int k0 = t * kBK;
    const __amdgpu_buffer_rsrc_t ww = window32(p.B + static_cast<int64_t>(k0) * p.ldb + n0,
                                               (static_cast<int64_t>(kend - k0 - 1) * p.ldb + (p.N - n0)) * 2);
#pragma unroll
    for (int i = 0; i < kWRows; ++i)
      r.w[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ww, w_off[i], 0, kCacheNT));
    const __amdgpu_buffer_rsrc_t wx =
        window32(p.A + k0, (static_cast<int64_t>(p.M - 1) * p.lda + (kend - k0)) * 2);
    r.x = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(wx, x_off | (k0 + 8 * xc < kend ? 0u : kOutOfRange), 0, 0));
  };
  auto store_slice = [&](int t, const SliceRegs& r) {
    uint8_t* st = smem + (t % NS) * kStage;
#pragma unroll
    for (int i = 0; i < kWRows; ++i)
      *reinterpret_cast<u32x4*>(st + (kWRows * wave + i) * kWRow + 16 * lane) = r.w[i];
    *reinterpret_cast<u32x4*>(st + kWStage + wave * 1024 + 16 * lane) = r.x;
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

  auto compute_slice = [&](int t) {
    const uint8_t* base = smem + (t % NS) * kStage;
    bf16x8 fb[kFN], fx[MB];
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, base + b_off[j]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, base + b_off[j] + 4 * kWRow));
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
  };
  if constexpr (REG) {
    // One slice: its registers go to LDS stage t % NS, the same registers
    // are refilled with slice t + 2, and after the barrier (stage t complete
    // in every wave; stage t - 1 no longer read) the slice is multiplied.
    // Two slices stay in flight per wave while the MFMAs run.
    auto step = [&](int t, SliceRegs& r) {
      store_slice(t, r);
      load_slice(t + 2, r);
      lds_barrier();
      compute_slice(t);
    };
    if (te > tb) {
      SliceRegs r0, r1;
      load_slice(tb, r0);
      load_slice(tb + 1, r1);
      int t = tb;
      for (; t + 1 < te; t += 2) {
        step(t, r0);
        step(t + 1, r1);
      }
      if (t < te) step(t, r0);
    }
  } else {
    // Direct buffer loads into LDS stage t % NS, NS - 1 slices in flight;
    // the same lane -> LDS placement as above.
    const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
    auto issue_slice = [&](int t) {
      const uint32_t stage = smem_base + static_cast<uint32_t>((t % NS) * kStage);
      const int k0 = t * kBK;
      const i32x4 ww = make_window_words(p.B + static_cast<int64_t>(k0) * p.ldb + n0,
                                         (static_cast<int64_t>(kend - k0 - 1) * p.ldb + (p.N - n0)) * 2);
#pragma unroll
      for (int i = 0; i < kWRows; ++i) buf_load16_lds(ww, stage + (kWRows * wave + i) * kWRow, w_off[i]);
      const i32x4 wx = make_window_words(p.A + k0, (static_cast<int64_t>(p.M - 1) * p.lda + (kend - k0)) * 2);
      buf_load16_lds(wx, stage + kWStage + wave * 1024, x_off | (k0 + 8 * xc < kend ? 0u : kOutOfRange));
    };
    if (te > tb) {
      for (int t = tb; t < tb + NS - 1; ++t) issue_slice(t);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * kLoadsPerSlice) : "memory");
      lds_barrier();
      for (int t = tb; t < te; ++t) {
        issue_slice(t + NS - 1);  // into the stage slice t-1 occupied
        compute_slice(t);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * kLoadsPerSlice) : "memory");
        lds_barrier();  // slice t+1 landed everywhere; slice t no longer read
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
    }
  }
}

// Stores 4 consecutive outputs v[0..3] of row `row` starting at column col
// (columns past N skipped).
template <bool OUT_BF16>
__device__ __forceinline__ void store4(const Bf16Args& p, int row, int col, const float (&v)[4]) {
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

template <int MB, int EPI, bool OUT_BF16, bool REG>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_thin(Bf16Args p) {
  apply_batch(p, OUT_BF16 ? 2 : 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[(REG ? kNSReg : kNSLds) * kStage];
  f32x4 acc[MB][kFN];
  thin_accumulate<MB, REG>(p, smem, acc);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kBN;

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
      store4<OUT_BF16>(p, row, col, v);
    }
  }
}

template <int MB, int EPI, bool OUT_BF16>
hipError_t launch_m(const Bf16Args& a, hipStream_t s) {
  const dim3 grid((a.N + kBN - 1) / kBN, a.batch);
  if (use_reg_pipeline(static_cast<int64_t>(grid.x) * grid.y))
    hipLaunchKernelGGL((tgemm_bf16_thin<MB, EPI, OUT_BF16, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((tgemm_bf16_thin<MB, EPI, OUT_BF16, false>), grid, dim3(kThreads), 0, s, a);
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

// ---- Split-K for small M and few column stripes ----
//
// With N = 4096 the thin kernel has only 8 workgroups for 256 compute units,
// and the weight stream stalls at a few percent of HBM bandwidth (up to
// 128 stripes, half the units or more sit idle).  The K
// range is then cut into S chunks (grid z): workgroup (stripe, s) sums
// slices [s*KTc, (s+1)*KTc) and writes its fp32 partial tile to
// part[s][M][N] (through the direct-to-LDS pipeline); a second kernel adds
// the S partials in order of s, then the bias and the epilogue, and rounds
// once -- deterministic, no atomics.
template <int MB>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_thin_splitk(Bf16Args p, float* part, int ktc) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNSLds * kStage];
  f32x4 acc[MB][kFN];
  const int KT = (p.K + kBK - 1) / kBK;
  const int tb = blockIdx.z * ktc;
  const int te = tb + ktc < KT ? tb + ktc : KT;
  thin_accumulate<MB, false>(p, smem, acc, tb, te);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kBN;
  Bf16Args pp = p;
  pp.C = part + static_cast<int64_t>(blockIdx.z) * p.M * p.N;
  pp.ldc = p.N;
  pp.vec_c = (p.N % 4) == 0 ? 1 : 0;
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int col = n0 + kWTN * wave + 16 * j + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + (lane & 15);
      if (row >= p.M) continue;
      const float v[4] = {acc[mb][j][0], acc[mb][j][1], acc[mb][j][2], acc[mb][j][3]};
      store4<false>(pp, row, col, v);
    }
  }
}

// Thread t of workgroup x handles the 4 outputs 4 (256 x + t) .. +3 of the
// row-major M x N result.
template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(256) void tgemm_splitk_reduce(Bf16Args p, const float* part, int S) {
  const int64_t i = 4 * (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
  const int64_t MN = static_cast<int64_t>(p.M) * p.N;
  if (i >= MN) return;
  const int row = static_cast<int>(i / p.N);
  const int col = static_cast<int>(i % p.N);
  // A 4-group never straddles rows when N % 4 == 0; otherwise go element-wise.
  const bool quad = (p.N % 4) == 0;
  float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < S; ++s) {
    const float* q = part + static_cast<int64_t>(s) * MN + i;
    if (quad) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(q);
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < MN) sum[e] += q[e];
    }
  }
  if (quad) {
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (EPI != kEpiNone) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bias[e] = bf16_bits_to_f32(p.bias[col + e]);
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = apply_epilogue<EPI>(sum[e], bias[e]);
    store4<OUT_BF16>(p, row, col, v);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i + e >= MN) break;
      const int r = static_cast<int>((i + e) / p.N), c = static_cast<int>((i + e) % p.N);
      const float b = EPI != kEpiNone ? bf16_bits_to_f32(p.bias[c]) : 0.0f;
      const float v = apply_epilogue<EPI>(sum[e], b);
      const int64_t off = static_cast<int64_t>(r) * p.ldc + c;
      if constexpr (OUT_BF16) static_cast<uint16_t*>(p.C)[off] = f32_to_bf16_bits(v);
      else static_cast<float*>(p.C)[off] = v;
    }
  }
}

template <int MB>
hipError_t launch_splitk_m(const Bf16Args& a, float* part, int S, int ktc, int epi, int out_bf16,
                           hipStream_t s) {
  hipLaunchKernelGGL((tgemm_bf16_thin_splitk<MB>), dim3((a.N + kBN - 1) / kBN, 1, S), dim3(kThreads), 0, s,
                     a, part, ktc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(a, part, S, epi, out_bf16, s);
}

// ---- Small-M GEMM with K-contiguous weights, Wt [N, K] (the nn.Linear
// layout of an LM head, [vocab, d_model]) ----
//
// Each output column is one contiguous weight row, so a workgroup owns 256
// rows of Wt (256 columns of C) and walks K in slices of 64: a slice of a
// row is one 128-byte cache line.  A load instruction brings 8 rows' lines
// (1 KiB); the same two pipelines as the [K, N] kernel, chosen the same way,
// take them to LDS (register-staged: two slices in flight per wave, two
// LDS stages, non-temporal weight loads; direct-to-LDS: four stages, three
// slices, 120 KiB, in flight).  Both MFMA operands are K-contiguous rows in LDS, read with one
// 16-byte read per lane (8 consecutive k); the 16-byte chunks of each
// 128-byte row are XOR-permuted by (row / 2) % 8 so the 16 rows one read
// covers land in 16 distinct bank slots.  Four waves each own 64 columns
// over all of K.
//
// Workgroup b walks its slices starting at slice 3b (mod the slice count).
// Weight rows (2K bytes apart, 8 KiB at K = 4096) read at one K offset by
// every workgroup at once concentrate on a few HBM channels; measured on
// the 4096 x 128256 head with direct-to-LDS loads, the staggered start takes
// the stream from 4.3 to 6.0 TB/s (the sum is the same, in a rotated order).
namespace nt {
constexpr int kBN = 256;        // weight rows (output columns) per workgroup
constexpr int kWTN = kBN / 4;   // per wave
constexpr int kFN = kWTN / 16;  // 16-column MFMA blocks per wave
constexpr int kBK = 64;         // K per slice
constexpr int kNSReg = 2;       // LDS stages, register-staged pipeline
constexpr int kNSLds = 4;       // LDS stages, direct-to-LDS pipeline
constexpr int kStagger = 3;     // first slice of workgroup b: kStagger * b (mod slices)
constexpr int kRow = kBK * 2;   // bytes per LDS row (weight or X)
constexpr int kChunks = kRow / 16;         // 16-byte chunks per row
constexpr int kRowsPerLoad = 1024 / kRow;  // rows one 1 KiB load covers
constexpr int kWStage = kBN * kRow;
constexpr int kXStage = 64 * kRow;       // 64 rows of X
constexpr int kStage = kWStage + kXStage;
constexpr int kWLoads = kWStage / 1024 / 4;  // per wave and slice
constexpr int kXLoads = kXStage / 1024 / 4;
constexpr int kLoadsPerSlice = kWLoads + kXLoads;
static_assert(kNSLds * kStage <= 160 * 1024, "LDS capacity");
// One slice of one wave in flight, 16 bytes per lane per load.
struct SliceRegs {
  u32x4 w[kWLoads];
  u32x4 x[kXLoads];
};
// 16 consecutive rows read at one logical chunk land in 16 distinct 16-byte
// bank slots.
__device__ __forceinline__ int swz(int r) {
  if constexpr (kChunks >= 16) return r & 15;
  else return (r >> 1) & 7;
}
}  // namespace nt

template <int MB, int EPI, bool OUT_BF16, bool REG>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_thin_nt(Bf16Args p) {
  constexpr int NS = REG ? nt::kNSReg : nt::kNSLds;
  apply_batch(p, OUT_BF16 ? 2 : 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * nt::kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * nt::kBN;

  f32x4 acc[MB][nt::kFN];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < nt::kFN; ++j) acc[mb][j] = f32x4{};

  // ---- global -> LDS: load i of wave w covers weight rows 64w + 8i ..
  // +7 of the stripe (lane l -> row l/8, physical chunk l%8, logical chunk
  // (l%8) ^ swz(row)); X loads cover rows 16w + 8i .. +7 the same way. ----
  const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  const int lr = lane / nt::kChunks, lc = lane % nt::kChunks;
  uint32_t w_off[nt::kWLoads];
  int w_kc[nt::kWLoads];
#pragma unroll
  for (int i = 0; i < nt::kWLoads; ++i) {
    const int r = nt::kWTN * wave + nt::kRowsPerLoad * i + lr;
    const int c = lc ^ nt::swz(r);
    w_off[i] = static_cast<uint32_t>(r * ldb2 + 16 * c);
    w_kc[i] = 8 * c;
  }
  uint32_t x_off[nt::kXLoads];
  int x_kc[nt::kXLoads];
#pragma unroll
  for (int i = 0; i < nt::kXLoads; ++i) {
    const int r = 16 * wave + nt::kRowsPerLoad * i + lr;
    const int c = lc ^ nt::swz(r);
    x_off[i] = static_cast<uint32_t>(r * lda2 + 16 * c);
    x_kc[i] = 8 * c;
  }
  const int KT = (p.K + nt::kBK - 1) / nt::kBK;
  const int t0 = KT > 0 ? static_cast<int>((static_cast<int64_t>(blockIdx.x) * nt::kStagger) % KT) : 0;
  // The t-th slice walked is slice (t0 + t) mod KT; t >= KT loads nothing
  // (k0 = K: every offset flagged out of range).  Weight rows n0 .. N-1 and
  // X rows 0 .. M-1 from column k0; rows past the ends and columns past K
  // read zeros.  Weight lines are read once by the whole grid and carry the
  // non-temporal hint; X is re-read by every workgroup and stays cacheable.
  auto load_slice = [&](int t, nt::SliceRegs& r) {
    const int k0 = t < KT ? (t0 + t < KT ? t0 + t : t0 + t - KT) * nt::kBK : p.K;
    const __amdgpu_buffer_rsrc_t ww = window32(p.B + static_cast<int64_t>(n0) * p.ldb + k0,
                                               (static_cast<int64_t>(p.N - n0 - 1) * p.ldb + (p.K - k0)) * 2);
#pragma unroll
    for (int i = 0; i < nt::kWLoads; ++i)
      r.w[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ww, w_off[i] | (k0 + w_kc[i] < p.K ? 0u : kOutOfRange), 0,
                                                       kCacheNT));
    const __amdgpu_buffer_rsrc_t wx =
        window32(p.A + k0, (static_cast<int64_t>(p.M - 1) * p.lda + (p.K - k0)) * 2);
#pragma unroll
    for (int i = 0; i < nt::kXLoads; ++i)
      r.x[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wx, x_off[i] | (k0 + x_kc[i] < p.K ? 0u : kOutOfRange), 0, 0));
  };
  // Lane l's 16 bytes of load i go to LDS at the load's first row + 16 l.
  auto store_slice = [&](int t, const nt::SliceRegs& r) {
    uint8_t* st = smem + (t % NS) * nt::kStage;
#pragma unroll
    for (int i = 0; i < nt::kWLoads; ++i)
      *reinterpret_cast<u32x4*>(st + (nt::kWTN * wave + nt::kRowsPerLoad * i) * nt::kRow + 16 * lane) = r.w[i];
#pragma unroll
    for (int i = 0; i < nt::kXLoads; ++i)
      *reinterpret_cast<u32x4*>(st + nt::kWStage + (16 * wave + nt::kRowsPerLoad * i) * nt::kRow + 16 * lane) =
          r.x[i];
  };

  // ---- LDS -> registers: operand of MFMA step u (K 32u .. 32u+31 of the
  // slice): lane l reads row (l%16) of its block, logical chunk 4u + l/16. ----
  const int l16 = lane & 15, lq = lane >> 4;
  const int w_rd = (nt::kWTN * wave + l16) * nt::kRow;  // + 16 j rows; swz(row) = swz(l16)
  const int x_rd = nt::kWStage + l16 * nt::kRow;  // + 16 mb rows
  const int sw = nt::swz(l16);
  auto compute_slice = [&](int t) {
    const uint8_t* base = smem + (t % NS) * nt::kStage;
#pragma unroll
    for (int u = 0; u < nt::kBK / 32; ++u) {
      const int ch = ((4 * u + lq) ^ sw) * 16;
      bf16x8 fw[nt::kFN], fx[MB];
#pragma unroll
      for (int j = 0; j < nt::kFN; ++j)
        fw[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + w_rd + 16 * j * nt::kRow + ch));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        fx[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + x_rd + 16 * mb * nt::kRow + ch));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < nt::kFN; ++j)
          acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fx[mb], acc[mb][j], 0, 0, 0);
    }
  };
  if constexpr (REG) {
    // As in the [K, N] kernel: slice t's registers go to LDS stage t % NS
    // and are refilled with slice t + 2; after the barrier slice t is
    // multiplied.
    auto step = [&](int t, nt::SliceRegs& r) {
      store_slice(t, r);
      load_slice(t + 2, r);
      lds_barrier();
      compute_slice(t);
    };
    if (KT > 0) {
      nt::SliceRegs r0, r1;
      load_slice(0, r0);
      load_slice(1, r1);
      int t = 0;
      for (; t + 1 < KT; t += 2) {
        step(t, r0);
        step(t + 1, r1);
      }
      if (t < KT) step(t, r0);
    }
  } else {
    // Direct buffer loads into LDS stage t % NS, NS - 1 slices in flight,
    // with the same lane -> LDS placement as store_slice.
    const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
    auto issue_slice = [&](int t) {
      const uint32_t stage = smem_base + static_cast<uint32_t>((t % NS) * nt::kStage);
      const int k0 = t < KT ? (t0 + t < KT ? t0 + t : t0 + t - KT) * nt::kBK : p.K;
      const i32x4 ww = make_window_words(p.B + static_cast<int64_t>(n0) * p.ldb + k0,
                                         (static_cast<int64_t>(p.N - n0 - 1) * p.ldb + (p.K - k0)) * 2);
#pragma unroll
      for (int i = 0; i < nt::kWLoads; ++i)
        buf_load16_lds(ww, stage + (nt::kWTN * wave + nt::kRowsPerLoad * i) * nt::kRow,
                       w_off[i] | (k0 + w_kc[i] < p.K ? 0u : kOutOfRange));
      const i32x4 wx = make_window_words(p.A + k0, (static_cast<int64_t>(p.M - 1) * p.lda + (p.K - k0)) * 2);
#pragma unroll
      for (int i = 0; i < nt::kXLoads; ++i)
        buf_load16_lds(wx, stage + nt::kWStage + (16 * wave + nt::kRowsPerLoad * i) * nt::kRow,
                       x_off[i] | (k0 + x_kc[i] < p.K ? 0u : kOutOfRange));
    };
    if (KT > 0) {
      for (int t = 0; t < NS - 1; ++t) issue_slice(t);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * nt::kLoadsPerSlice) : "memory");
      lds_barrier();
      for (int t = 0; t < KT; ++t) {
        issue_slice(t + NS - 1);  // into the stage slice t-1 occupied
        compute_slice(t);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * nt::kLoadsPerSlice) : "memory");
        lds_barrier();  // slice t+1 landed everywhere; slice t no longer read
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
    }
  }

  // ---- epilogue: element e of lane l in block (mb, j) is row 16 mb + l%16,
  // column 16 j + 4 (l/16) + e of the wave's 64 ----
#pragma unroll
  for (int j = 0; j < nt::kFN; ++j) {
    const int col = n0 + nt::kWTN * wave + 16 * j + 4 * lq;
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (EPI != kEpiNone) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < p.N) bias[e] = bf16_bits_to_f32(p.bias[col + e]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + l16;
      if (row >= p.M) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = apply_epilogue<EPI>(acc[mb][j][e], bias[e]);
      store4<OUT_BF16>(p, row, col, v);
    }
  }
}

template <int MB, int EPI, bool OUT_BF16>
hipError_t launch_nt_m(const Bf16Args& a, hipStream_t s) {
  const dim3 grid((a.N + nt::kBN - 1) / nt::kBN, a.batch);
  if (use_reg_pipeline(static_cast<int64_t>(grid.x) * grid.y))
    hipLaunchKernelGGL((tgemm_bf16_thin_nt<MB, EPI, OUT_BF16, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((tgemm_bf16_thin_nt<MB, EPI, OUT_BF16, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MB>
hipError_t dispatch_nt_epi(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (out_bf16) {
    if (epi == kEpiNone) return launch_nt_m<MB, kEpiNone, true>(a, s);
    if (epi == kEpiBias) return launch_nt_m<MB, kEpiBias, true>(a, s);
    return launch_nt_m<MB, kEpiBiasGelu, true>(a, s);
  }
  if (epi == kEpiNone) return launch_nt_m<MB, kEpiNone, false>(a, s);
  if (epi == kEpiBias) return launch_nt_m<MB, kEpiBias, false>(a, s);
  return launch_nt_m<MB, kEpiBiasGelu, false>(a, s);
}

// ---- LM head with bias and log-softmax over each row (GEMM compute-cost
// page, section 7.2: the output GEMM, its bias add and the LogSoftmax that
// follows, fused) ----
//
//   out[i, n] = y[i, n] - lse_i,  y = X W + bias,  lse_i = log sum_n exp(y[i, n])
//
// Pass 1 (the thin GEMM's epilogue): each workgroup adds the bias to its
// stripe's logits, forms per row the stripe maximum m_w and s_w =
// sum exp(y - m_w) (the safe-softmax pair) and writes them to part[row * G +
// w], and writes the fp32 logits (into C for fp32 output, else into the
// workspace, so each output is rounded once).  Pass 2 (lsm_normalize) merges
// the G pairs of a row, lse = m + log s with m = max_w m_w and s =
// sum_w s_w exp(m_w - m), and writes y - lse.  The logits cross HBM once
// each way (3-4 bytes per output per pass, small beside the weight the
// first pass streams); a single pass would need a grid-wide barrier.

// Merges the pair (m2, s2) into (m, s); m == -inf marks an empty pair.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -__builtin_inff()) return;
  if (m == -__builtin_inff()) {
    m = m2;
    s = s2;
    return;
  }
  const float mn = __builtin_fmaxf(m, m2);
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

template <int MB, bool REG>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_thin_lsm(Bf16Args p, LsmArgs q) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[(REG ? kNSReg : kNSLds) * kStage];
  f32x4 acc[MB][kFN];
  thin_accumulate<MB, REG>(p, smem, acc);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kBN;
  constexpr float kNegInf = -__builtin_inff();

  // Logits with bias; columns past N take -inf, which no maximum or sum sees.
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int col = n0 + kWTN * wave + 16 * j + 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = col + e < p.N;
      const float b = (in && p.bias != nullptr) ? bf16_bits_to_f32(p.bias[col + e]) : 0.0f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][j][e] = in ? acc[mb][j][e] + b : kNegInf;
    }
  }

  // Row 16 mb + l%16 of the stripe: lanes l, l^16, l^32, l^48 of each wave
  // hold its columns; the four waves meet in LDS.
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][64 rows]
  __syncthreads();  // every wave's loads have landed: smem is free
  float mrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = __builtin_fmaxf(m, acc[mb][j][e]);
    m = __builtin_fmaxf(m, __shfl_xor(m, 16, 64));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
    if (lane < 16) red[wave * 64 + 16 * mb + lane] = m;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = 16 * mb + (lane & 15);
    mrow[mb] = __builtin_fmaxf(__builtin_fmaxf(red[r], red[64 + r]), __builtin_fmaxf(red[128 + r], red[192 + r]));
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) t += __expf(acc[mb][j][e] - mrow[mb]);
    t += __shfl_xor(t, 16, 64);
    t += __shfl_xor(t, 32, 64);
    if (lane < 16) red[wave * 64 + 16 * mb + lane] = t;
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = 16 * mb + lane;
      const float srow = (red[r] + red[64 + r]) + (red[128 + r] + red[192 + r]);
      if (r < p.M) q.part[static_cast<int64_t>(r) * gridDim.x + blockIdx.x] = float2{mrow[mb], srow};
    }
  }

  // fp32 logits to their buffer.
  Bf16Args pl = p;
  pl.C = q.logits;
  pl.ldc = q.ldl;
  pl.vec_c = q.vec_l;
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int col = n0 + kWTN * wave + 16 * j + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + (lane & 15);
      if (row >= p.M) continue;
      const float v[4] = {acc[mb][j][0], acc[mb][j][1], acc[mb][j][2], acc[mb][j][3]};
      store4<false>(pl, row, col, v);
    }
  }
}

// Pass 2: workgroup (x, y) normalises columns kChunk x .. + kChunk - 1 of
// row y; each thread takes 16 columns, as four 4-column groups 1 KiB apart
// per wave.
constexpr int kChunk = 4096;

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void tgemm_lsm_normalize(LsmArgs q, void* C, int64_t ldc, int N,
                                                           int vec_c) {
  __shared__ float red[2][4];
  const int r = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int G = q.G;
  float m = -__builtin_inff(), s = 0.0f;
  const float2* part = q.part + static_cast<int64_t>(r) * G;
  for (int w = t; w < G; w += 256) {
    const float2 v = part[w];
    lse_merge(m, s, v.x, v.y);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float m2 = __shfl_xor(m, d, 64);
    const float s2 = __shfl_xor(s, d, 64);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    red[0][wave] = m;
    red[1][wave] = s;
  }
  __syncthreads();
  m = red[0][0];
  s = red[1][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_merge(m, s, red[0][w], red[1][w]);
  const float lse = m + __logf(s);

  const float* lrow = q.logits + static_cast<int64_t>(r) * q.ldl;
  Bf16Args po{};
  po.C = C;
  po.ldc = ldc;
  po.N = N;
  po.vec_c = vec_c;
#pragma unroll
  for (int i = 0; i < kChunk / 1024; ++i) {
    const int col = blockIdx.x * kChunk + 1024 * i + 4 * t;
    if (col >= N) break;
    float v[4];
    if (q.vec_l && col + 4 <= N) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(lrow + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[e] - lse;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = col + e < N ? lrow[col + e] - lse : 0.0f;
    }
    store4<OUT_BF16>(po, r, col, v);
  }
}

template <int MB>
hipError_t launch_lsm_m(const Bf16Args& a, const LsmArgs& q, hipStream_t s) {
  if (use_reg_pipeline(q.G))
    hipLaunchKernelGGL((tgemm_bf16_thin_lsm<MB, true>), dim3(q.G), dim3(kThreads), 0, s, a, q);
  else
    hipLaunchKernelGGL((tgemm_bf16_thin_lsm<MB, false>), dim3(q.G), dim3(kThreads), 0, s, a, q);
  return hipGetLastError();
}

}  // namespace

int64_t lsm_workgroups(int64_t N) { return (N + kBN - 1) / kBN; }

bool lsm_direct_ok(const Bf16Args& a) {
  return a.M <= 64 && a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
         a.ldb * 2 * kBK < (int64_t{1} << 31) && a.lda * 2 * 64 < (int64_t{1} << 31);
}

hipError_t launch_lsm_normalize(const LsmArgs& q, void* C, int64_t ldc, int M, int N, int vec_c,
                                int out_bf16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((N + kChunk - 1) / kChunk), static_cast<unsigned>(M));
  if (out_bf16)
    hipLaunchKernelGGL((tgemm_lsm_normalize<true>), grid, dim3(256), 0, s, q, C, ldc, N, vec_c);
  else
    hipLaunchKernelGGL((tgemm_lsm_normalize<false>), grid, dim3(256), 0, s, q, C, ldc, N, vec_c);
  return hipGetLastError();
}

hipError_t launch_bf16_thin_lsm(const Bf16Args& a, const LsmArgs& q, int out_bf16, hipStream_t s) {
  hipError_t e;
  if (a.M <= 16) e = launch_lsm_m<1>(a, q, s);
  else if (a.M <= 32) e = launch_lsm_m<2>(a, q, s);
  else if (a.M <= 48) e = launch_lsm_m<3>(a, q, s);
  else e = launch_lsm_m<4>(a, q, s);
  if (e != hipSuccess) return e;
  return launch_lsm_normalize(q, a.C, a.ldc, a.M, a.N, a.vec_c, out_bf16, s);
}

ThinSplit thin_split_plan(int64_t M, int64_t N, int64_t K) {
  // Enough (stripe, chunk) workgroups to cover the compute units, chunks of
  // at least 4 slices, and partial traffic (2 S M N fp32) at most half the
  // weight's bytes (2 K N): S <= K / (8 M).
  ThinSplit r{1, 0};
  const int64_t stripes = (N + kBN - 1) / kBN;
  const int64_t KT = (K + kBK - 1) / kBK;
  if (M < 1 || stripes > 128 || KT < 8) return r;  // over half the units busy: no split
  int64_t S = (256 + stripes - 1) / stripes;
  S = S < KT / 4 ? S : KT / 4;
  const int64_t cap = K / (8 * M);
  S = S < cap ? S : cap;
  if (S < 2) return r;
  const int64_t ktc = (KT + S - 1) / S;
  r.S = static_cast<int>((KT + ktc - 1) / ktc);
  r.ktc = static_cast<int>(ktc);
  return r;
}

hipError_t launch_splitk_reduce(const Bf16Args& a, const float* part, int S, int epi, int out_bf16,
                                hipStream_t s) {
  const int64_t quads = (static_cast<int64_t>(a.M) * a.N + 3) / 4;
  const dim3 grid(static_cast<unsigned>((quads + 255) / 256));
  if (out_bf16) {
    if (epi == kEpiNone) hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiNone, true>), grid, dim3(256), 0, s, a, part, S);
    else if (epi == kEpiBias) hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiBias, true>), grid, dim3(256), 0, s, a, part, S);
    else hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiBiasGelu, true>), grid, dim3(256), 0, s, a, part, S);
  } else {
    if (epi == kEpiNone) hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiNone, false>), grid, dim3(256), 0, s, a, part, S);
    else if (epi == kEpiBias) hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiBias, false>), grid, dim3(256), 0, s, a, part, S);
    else hipLaunchKernelGGL((tgemm_splitk_reduce<kEpiBiasGelu, false>), grid, dim3(256), 0, s, a, part, S);
  }
  return hipGetLastError();
}

hipError_t launch_bf16_thin_splitk(const Bf16Args& a, const ThinSplit& plan, float* part, int epi,
                                   int out_bf16, hipStream_t s) {
  if (a.M <= 16) return launch_splitk_m<1>(a, part, plan.S, plan.ktc, epi, out_bf16, s);
  if (a.M <= 32) return launch_splitk_m<2>(a, part, plan.S, plan.ktc, epi, out_bf16, s);
  if (a.M <= 48) return launch_splitk_m<3>(a, part, plan.S, plan.ktc, epi, out_bf16, s);
  return launch_splitk_m<4>(a, part, plan.S, plan.ktc, epi, out_bf16, s);
}

bool thin_nt_ok(const Bf16Args& a) {
  return a.M <= 64 && a.vec_a && a.vec_b && a.K % 8 == 0 &&
         a.ldb * 2 * nt::kBN < (int64_t{1} << 31) && a.lda * 2 * 64 < (int64_t{1} << 31);
}

hipError_t launch_bf16_thin_nt(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (a.M <= 16) return dispatch_nt_epi<1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_nt_epi<2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_nt_epi<3>(a, epi, out_bf16, s);
  return dispatch_nt_epi<4>(a, epi, out_bf16, s);
}

const char* thin_kernel_name(int M, bool split) {
  if (split) {
    if (M <= 16) return "tgemm_bf16_thin_splitk_m16+tgemm_splitk_reduce";
    if (M <= 32) return "tgemm_bf16_thin_splitk_m32+tgemm_splitk_reduce";
    if (M <= 48) return "tgemm_bf16_thin_splitk_m48+tgemm_splitk_reduce";
    return "tgemm_bf16_thin_splitk_m64+tgemm_splitk_reduce";
  }
  if (M <= 16) return "tgemm_bf16_thin_m16";
  if (M <= 32) return "tgemm_bf16_thin_m32";
  if (M <= 48) return "tgemm_bf16_thin_m48";
  return "tgemm_bf16_thin_m64";
}

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // Once per device, with that device current (it is the caller's current
  // device): the device address of this device's copy of the array.
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool thin_direct_ok(const Bf16Args& a) {
  // Direct loads need 16-byte aligned rows and per-lane offsets below 2^31
  // (a slice's 32 rows of W, 64 rows of X).
  return a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
         a.ldb * 2 * kBK < (int64_t{1} << 31) && a.lda * 2 * 64 < (int64_t{1} << 31);
}

int64_t thin_split_bytes(const ThinSplit& plan, int64_t M, int64_t N) {
  return plan.S > 1 ? static_cast<int64_t>(plan.S) * M * N * 4 : 0;
}

hipError_t launch_bf16_thin(const Bf16Args& a, int epi, int out_bf16, hipStream_t s, float* part,
                            int64_t part_bytes) {
  if (!thin_direct_ok(a)) return launch_bf16_thin_general(a, epi, out_bf16, s);
  if (a.batch == 1 && part != nullptr) {
    const ThinSplit plan = thin_split_plan(a.M, a.N, a.K);
    if (plan.S > 1 && part_bytes >= thin_split_bytes(plan, a.M, a.N))
      return launch_bf16_thin_splitk(a, plan, part, epi, out_bf16, s);
  }
  if (a.M <= 16) return dispatch_epi<1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_epi<2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_epi<3>(a, epi, out_bf16, s);
  return dispatch_epi<4>(a, epi, out_bf16, s);
}

}  // namespace tgemm
