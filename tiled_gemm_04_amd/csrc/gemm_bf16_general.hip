// General-layout bf16 GEMM for gfx950: C = epilogue(A . B + bias), fp32
// accumulate, for operands the direct-to-LDS kernel cannot take (row strides
// or base addresses that are not 16-byte multiples, inner extents that are not
// multiples of 8, offsets that do not fit the 32-bit buffer range).
//
// Structure (DeepGEMM page, sections 2.1-2.3; tensor-core page, "Chunking"):
// each workgroup owns one BM x BN tile and walks K in slices of 64; A and B
// chunks are assembled element by element with bounds checks (zero outside M,
// N, K: DeepGEMM page, section 4.1), staged in registers and written to LDS
// (B transposed 8 x 8 on the way, so both operands sit K-contiguous); two LDS
// stages, with the MFMA operands of sub-step s+1 read while the MFMAs of
// sub-step s run.  The epilogue (bias, tanh-GeLU, rounding: GEMM compute-cost
// page, section 5.1) goes through LDS and masks every store.
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
  // Epilogue staging: one 32-row strip of a wave's tile in fp32, rows padded
  // by 16 bytes.
  static constexpr int EPI_PITCH = WTN + 4;
  static constexpr int EPI_LANES_PER_ROW = WTN / 8;
  static constexpr int EPI_ROWS_PER_PASS = kWave / EPI_LANES_PER_ROW;
  static_assert((BM * 8) % kThreads == 0, "A slice must split evenly over the threads");
  static_assert(BN <= kThreads, "one thread per 8 x 8 block of the B slice");
  static_assert(FM >= 2 && FN >= 1, "wave tile must hold two 32-row MFMA blocks");
  static_assert(4 * 32 * EPI_PITCH * 4 <= LDS_SLOTS * 16, "epilogue staging must fit in LDS");
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

template <class T, int EPI, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void tgemm_bf16_general(Bf16Args p, int tiles_m,
                                                                int tiles_n) {
  apply_batch(p, OUT_BF16 ? 2 : 4);
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

  // acc[i][j] holds the transposed 32 x 32 block (MFMA operands swapped):
  // element 4*g + e of lane l is row 32*i + l%32, column 32*j + 8*g + 4*(l/32) + e.
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
  constexpr bool kAllOwnB = T::B_THREADS == kThreads;
  const bool b_owner = kAllOwnB || tid < T::B_THREADS;

  u32x4 ra[T::A_PER_THREAD];
  u32x4 rb[8];

  // One bounds-checked 16-byte chunk of A (chunk i) or B (row r of the 8 x 8
  // block) for the slice starting at k0.
  auto gload_a = [&](int k0, int i) {
    ra[i] = load16_checked(p.A, p.lda, m0 + a_r + 32 * i, p.M, k0 + 8 * a_c, p.K);
  };
  auto gload_b = [&](int k0, int r) {
    if (b_owner) rb[r] = load16_checked(p.B, p.ldb, k0 + 8 * b_kb + r, p.K, n0 + 8 * b_nb, p.N);
  };
  // One 16-byte LDS write: A chunk i, or column j of the transposed B block.
  auto sstore_a = [&](int stage, int i) {
    sA[stage * T::A_STAGE + a_c * T::BM + (a_r ^ a_c) + 32 * i] = ra[i];
  };
  auto sstore_b = [&](int stage, int j) {
    if (b_owner) sB[stage * T::B_STAGE + b_kb * T::BN + 8 * b_nb + (j ^ b_kb)] = transpose_col(rb, j);
  };

  // MFMA operands of one 16-wide K sub-step, double-buffered in registers:
  // fragment f < FM is A block f, the rest are B blocks.
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  constexpr int kNR = T::FM + T::FN;
  bf16x8 fa[2][T::FM], fb[2][T::FN];
  auto lds_read = [&](int buf, int stage, int ks, int f) {
    const int c = 2 * ks + lhalf;
    if (f < T::FM) {
      fa[buf][f] = __builtin_bit_cast(
          bf16x8, sA[stage * T::A_STAGE + c * T::BM + ((wm * T::WTM + lrow) ^ c) + 32 * f]);
    } else {
      fb[buf][f - T::FM] = __builtin_bit_cast(
          bf16x8,
          sB[stage * T::B_STAGE + c * T::BN + ((wn * T::WTN + lrow) ^ c) + 32 * (f - T::FM)]);
    }
  };
  // MFMA for accumulator block q = i * FN + j.
  constexpr int kQ = T::FM * T::FN;
  auto mfma_one = [&](int buf, int q) {
    const int i = q / T::FN, j = q % T::FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };

  // Slot schedule of one slice t (stage cur holds it, stage cur^1 is idle).
  // The slice is 4 sub-steps of kQ MFMAs (slots 0 .. 4kQ-1); every other
  // instruction is spread over the MFMA slots so that the single wave per
  // SIMD never stalls the matrix unit for long:
  //   [0, kQ/2)        read operands of sub-step 1
  //   [kQ/2, kQ)       A registers of slice t+1 -> stage cur^1
  //   [kQ, 3kQ/2)      read operands of sub-step 2; A loads of slice t+2
  //   [3kQ/2, 2kQ)     B registers of slice t+1 -> stage cur^1 (transposed)
  //   [2kQ, 5kQ/2)     read operands of sub-step 3; B loads of slice t+2
  //   barrier before slot 3kQ (stage cur fully read, stage cur^1 written)
  //   [3kQ, 7kQ/2)     read operands of sub-step 0 of slice t+1
  // A global load therefore has almost a whole slice to arrive before its
  // register is written to LDS.  (The fast path of aligned operands is the
  // direct-to-LDS kernel; this one only has to be correct and not slow.)
  const int KT = (p.K + kBK - 1) / kBK;
  if (KT > 0) {
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) gload_a(0, i);
#pragma unroll
    for (int r = 0; r < 8; ++r) gload_b(0, r);
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) sstore_a(0, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) sstore_b(0, j);
    // Slice 1; past K the checked loads return zeros.
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) gload_a(kBK, i);
#pragma unroll
    for (int r = 0; r < 8; ++r) gload_b(kBK, r);
    lds_barrier();
#pragma unroll
    for (int f = 0; f < kNR; ++f) lds_read(0, 0, 0, f);
    for (int t = 0; t < KT; ++t) {
      const int cur = t & 1;
      const int k2 = (t + 2) * kBK;
      static_for<4 * kQ>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 3 * kQ) {
          TGEMM_SCHED_FENCE();
          lds_barrier();
        }
        TGEMM_SCHED_FENCE();
        mfma_one((s / kQ) & 1, s % kQ);
        TGEMM_SCHED_FENCE();
        static_for<kNR>([&](auto fc) {
          constexpr int f = decltype(fc)::value;
          if constexpr (spread(f, kNR, 0, kQ / 2) == s) lds_read(1, cur, 1, f);
          if constexpr (spread(f, kNR, kQ, 3 * kQ / 2) == s) lds_read(0, cur, 2, f);
          if constexpr (spread(f, kNR, 2 * kQ, 5 * kQ / 2) == s) lds_read(1, cur, 3, f);
          if constexpr (spread(f, kNR, 3 * kQ, 7 * kQ / 2) == s) lds_read(0, cur ^ 1, 0, f);
        });
        static_for<T::A_PER_THREAD>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (spread(i, T::A_PER_THREAD, kQ / 2, kQ) == s) sstore_a(cur ^ 1, i);
          if constexpr (spread(i, T::A_PER_THREAD, kQ, 3 * kQ / 2) == s) gload_a(k2, i);
        });
        static_for<8>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          if constexpr (spread(r, 8, 3 * kQ / 2, 2 * kQ) == s) sstore_b(cur ^ 1, r);
          if constexpr (spread(r, 8, 2 * kQ, 5 * kQ / 2) == s) gload_b(k2, r);
        });
      });
      TGEMM_SCHED_FENCE();
    }
  }
  lds_barrier();  // every wave is done with the operand stages

  // ---- epilogue: one 32-row strip at a time through this wave's LDS area ----
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * T::EPI_PITCH;
  const int erow = lane / T::EPI_LANES_PER_ROW;
  const int ecol = 8 * (lane % T::EPI_LANES_PER_ROW);
  const int gcol = n0 + wn * T::WTN + ecol;
  float bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bias[e] = 0.0f;
    if constexpr (EPI != kEpiNone) {
      if (gcol + e < p.N) bias[e] = bf16_bits_to_f32(p.bias[gcol + e]);
    }
  }
  const bool full_cols = p.vec_c && gcol + 8 <= p.N;

#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(stage + lrow * T::EPI_PITCH + 32 * j + 8 * g + 4 * lhalf) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                  acc[i][j][4 * g + 3]};
#pragma unroll
    for (int pass = 0; pass < 32 / T::EPI_ROWS_PER_PASS; ++pass) {
      const int rr = erow + T::EPI_ROWS_PER_PASS * pass;
      const float* src = stage + rr * T::EPI_PITCH + ecol;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_epilogue<EPI>(v[e], bias[e]);
      const int row = m0 + wm * T::WTM + 32 * i + rr;
      if (row < p.M) {
        const int64_t off = static_cast<int64_t>(row) * p.ldc + gcol;
        if constexpr (OUT_BF16) {
          uint16_t* out = static_cast<uint16_t*>(p.C) + off;
          if (full_cols) {
            *reinterpret_cast<u32x4*>(out) =
                u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gcol + e < p.N) out[e] = f32_to_bf16_bits(v[e]);
          }
        } else {
          float* out = static_cast<float*>(p.C) + off;
          if (full_cols) {
            *reinterpret_cast<f32x4*>(out) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(out + 4) = f32x4{v[4], v[5], v[6], v[7]};
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gcol + e < p.N) out[e] = v[e];
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
  hipLaunchKernelGGL((tgemm_bf16_general<T, EPI, OUT_BF16>), dim3(tiles_m * tiles_n, a.batch),
                     dim3(kThreads), 0, s, a, tiles_m, tiles_n);
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

hipError_t launch_bf16_general(const Bf16Args& a, int shape, int epi, int out_bf16,
                               hipStream_t s) {
  switch (shape) {
    case kTile256x256: return dispatch_epi<Tiled<256, 256>>(a, epi, out_bf16, s);
    case kTile256x128: return dispatch_epi<Tiled<256, 128>>(a, epi, out_bf16, s);
    default: return dispatch_epi<Tiled<128, 128>>(a, epi, out_bf16, s);
  }
}

}  // namespace tgemm
