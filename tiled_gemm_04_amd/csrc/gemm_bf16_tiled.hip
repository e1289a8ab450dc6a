// Direct-to-LDS bf16 GEMM for gfx950: C = epilogue(A . B + bias), fp32 accumulate.
//
// The method (DeepGEMM page, sections 2.1-2.3 and 3.3; tensor-core page,
// "Chunking" and "Registers与Tensor Cores") maps onto CDNA4 as follows:
//   * tiling -- each workgroup owns one BM x BN output tile and walks K in
//     slices of BK; the waves split the tile 2 (along M) x WN (along N), each
//     owning a (BM/2) x (BN/WN) block of MFMA accumulator blocks held in
//     registers (256 x 256: eight waves, two per SIMD, 128 x 64 each, in
//     16 x 16 blocks of v_mfma_f32_16x16x32_bf16; the smaller tiles: four
//     waves, 2 x 2, in 32 x 32 blocks of v_mfma_f32_32x32x16_bf16);
//   * global -> LDS -- 16-byte buffer loads write straight into LDS (no
//     register staging, no LDS store instructions).  Each wave instruction
//     fills one contiguous KiB of LDS, lane l owning bytes 16l .. 16l+15, so
//     the layout is chosen by which global chunk each lane fetches.  A rows
//     (K-contiguous) and B rows (N-contiguous) are kept as they are in memory,
//     with the 16-byte chunks of each row permuted by an XOR of the row index
//     so that the MFMA operand reads below hit distinct LDS banks;
//   * LDS -> registers -- A operands with one 16-byte read per lane; B
//     operands with the gfx950 transposed read (ds_read_b64_tr_b16): within
//     each group of 16 lanes, lane 4e+q supplies 4 consecutive columns of K
//     row e and lane i receives column i of those 4 rows, i.e. 4 consecutive
//     k of one n -- the K-contiguous operand layout MFMA wants, read from an
//     N-contiguous tile (two reads per 8-k operand);
//   * pipelining -- NS LDS stages: the loads of slice t+NS-1 are issued while
//     slice t is multiplied, MFMA operands are double-buffered in registers,
//     and every non-MFMA instruction is placed between MFMAs by a
//     compile-time slot schedule, so that no burst of other instructions
//     leaves the matrix unit idle;
//   * epilogue -- bias, tanh-GeLU and output rounding applied to the fp32
//     accumulators (GEMM compute-cost page, section 5.1), the tile routed
//     through LDS so each lane stores 16 contiguous bytes; stores past M, N
//     are masked, and loads past M, N, K read zero through the buffer range
//     check (DeepGEMM page, section 4.1).
//
// B comes in either layout: [K, N] (N-contiguous, read with the transposed
// LDS reads above) or, with BT, [N, K] (K-contiguous, the nn.Linear weight
// layout) -- then B tiles are stored and read exactly like A tiles (plain
// 16-byte operand reads, the A swizzle).
//
// Requirements (checked by the launcher, otherwise the general kernel runs,
// or for BT the call is unsupported): A, B 16-byte aligned; lda, ldb
// multiples of 8; K multiple of 8 and (for [K, N] B) N multiple of 8; all
// per-lane byte offsets below 2^31.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kGroupM = 4;  // tile-rows per scheduling group

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int BM_, int BN_, int BK_, int NS_, int SPREAD_ = 1, int WN_ = 2, int MF_ = 32, int BAR_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_;
  // MFMA shape: 32 (v_mfma_f32_32x32x16_bf16, two K sub-steps per 32-wide
  // slice) or 16 (v_mfma_f32_16x16x32_bf16, one per 32-wide slice).
  static constexpr int MF = MF_;
  // 16 x 16 x 32 kernel: the slot before which each slice's barrier sits.
  static constexpr int BAR = BAR_;
  // Waves: 2 along M times WN along N (WN = 4: two waves per SIMD).
  static constexpr int WN = WN_;
  static constexpr int WAVES = 2 * WN;
  static constexpr int THREADS = 64 * WAVES;
  // Loads of a slice are spread over the first KS*FM*FN/SPREAD MFMA slots.
  static constexpr int SPREAD = SPREAD_;
  static constexpr int WTM = BM / 2, WTN = BN / WN;  // wave tile
  static constexpr int FM = WTM / MF, FN = WTN / MF;
  static constexpr int KS = BK / (MF == 32 ? 16 : 32);  // MFMA sub-steps per slice
  // A stage: BM rows of BK bf16 (A_CPR chunks of 16 bytes each).
  static constexpr int A_ROW = BK * 2;
  static constexpr int A_CPR = BK / 8;
  static constexpr int A_STAGE = BM * A_ROW;
  // B stage: BK rows of BN bf16.
  static constexpr int B_ROW = BN * 2;
  static constexpr int B_CPR = BN / 8;
  static constexpr int B_STAGE = BK * B_ROW;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int LDS_BYTES = NS * STAGE;
  // 1 KiB load blocks per wave and slice.
  static constexpr int APW = A_STAGE / 1024 / WAVES;
  static constexpr int BPW = B_STAGE / 1024 / WAVES;
  static constexpr int LPS = APW + BPW;  // loads per thread per slice
  // Epilogue staging: one 32-row strip of a wave's tile in fp32, rows padded by 16 bytes.
  static constexpr int EPI_PITCH = WTN + 4;
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  static_assert(BN >= 128, "the B-row swizzle needs at least 16 chunks per row");
  static_assert(MF == 32 || MF == 16, "MFMA shape");
  static_assert(MF == 32 || BK == 32, "the 16 x 16 x 32 kernel takes 32-wide slices");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold an MFMA block");
  static_assert(A_STAGE % (1024 * WAVES) == 0 && B_STAGE % (1024 * WAVES) == 0,
                "stages must split into 1 KiB loads per wave");
  static_assert(NS >= 2, "at least two stages");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
  static_assert(WAVES * 32 * EPI_PITCH * 4 <= LDS_BYTES, "epilogue staging must fit in LDS");
};

// XOR applied to the 16-byte chunk index of A row r (and of B row n for a
// K-contiguous B).  32 x 32 x 16 reads (lane 32h + r takes one chunk of row
// r < 32): consecutive rows that share a 256-byte LDS bank row get
// different permutations, so 16 lanes reading one chunk column of 16
// consecutive rows touch 16 distinct bank groups.  16 x 16 x 32 reads with
// 64-byte rows (lane 16q + r takes chunk q of row r < 16) were measured on
// MI355X over every XOR that is linear in the bits of r: the pattern above
// costs 2.15 ns per ds_read_b128 per compute unit, (r & 3) ^ 3 r[2] ^ 2 r[3]
// 1.43 ns, the fastest measured.  Both depend on r mod 16 only, so row
// blocks 16 apart share them.
template <class C>
__device__ __forceinline__ int a_swz(int r) {
  if constexpr (C::MF == 16 && C::A_CPR == 4) return (r & 3) ^ (3 * ((r >> 2) & 1)) ^ (2 * ((r >> 3) & 1));
  else return (r / (16 / C::A_CPR)) % C::A_CPR;
}
// XOR applied to the chunk index of B row k.  The four K rows read together
// by a transposed read land in four different 64-byte bank segments.  The
// 16 x 16 x 32 kernel's reads also put rows k and k + 8 in one half-wave:
// flipping chunk bit 1 with bit 3 of k moves those apart (SQ_LDS_BANK_CONFLICT
// on the 4096^3 GEMM: 25 % of LDS-active cycles without it, 1.9 % with it).
template <class C>
__device__ __forceinline__ int b_swz(int k) {
  if constexpr (C::MF == 16) return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1));
  else return 4 * (k & 3);
}

// Stores 8 consecutive outputs v of one row, columns gcol .. gcol+7 (those
// below N), rounded to bf16 or as fp32: one 16-byte store (two for fp32)
// when full_cols (aligned row, all 8 inside N), an unaligned one when the
// row is not 16-byte aligned, element stores at the right edge.
template <bool OUT_BF16>
__device__ __forceinline__ void store_row8(const float (&v)[8], int row, int gcol, bool full_cols,
                                           const Bf16Args& p) {
  const int64_t off = static_cast<int64_t>(row) * p.ldc + gcol;
  if constexpr (OUT_BF16) {
    uint16_t* out = static_cast<uint16_t*>(p.C) + off;
    if (full_cols) {
      // C is written once and not read back here: non-temporal stores
      // (measured 0.5-1.3 % faster on the tiled GEMMs).
      __builtin_nontemporal_store(
          u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
          reinterpret_cast<u32x4*>(out));
    } else if (gcol + 8 <= p.N) {
      // Row not 16-byte aligned: one unaligned 16-byte store.
      *reinterpret_cast<u32x4_a2*>(out) = u32x4_a2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gcol + e < p.N) out[e] = f32_to_bf16_bits(v[e]);
    }
  } else {
    float* out = static_cast<float*>(p.C) + off;
    if (full_cols) {
      __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(out));
      __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(out + 4));
    } else if (gcol + 8 <= p.N) {
      *reinterpret_cast<f32x4_a4*>(out) = f32x4_a4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4_a4*>(out + 4) = f32x4_a4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (gcol + e < p.N) out[e] = v[e];
    }
  }
}

// Epilogue of one wave: its FM x FN accumulator blocks (transposed 32 x 32
// layout, see the kernels) go through a private LDS strip of 32 rows, one
// strip at a time, so that every lane stores 8 consecutive outputs (16 bytes
// of bf16); bias, tanh-GeLU and rounding are applied on the way out
// (GEMM compute-cost page, section 5.1).  row0 / col0: the wave tile's first
// output row / column.  Rows >= M and columns >= N are not stored.
template <int EPI, bool OUT_BF16, int FM, int FN>
__device__ __forceinline__ void store_wave_tile(const f32x16 (&acc)[FM][FN], float* strip, int lane,
                                                int row0, int col0, const Bf16Args& p) {
  constexpr int WTN = 32 * FN;
  constexpr int PITCH = WTN + 4;  // floats; 16 bytes of padding per row
  constexpr int LANES_PER_ROW = WTN / 8;
  constexpr int ROWS_PER_PASS = kWave / LANES_PER_ROW;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int erow = lane / LANES_PER_ROW;
  const int ecol = 8 * (lane % LANES_PER_ROW);
  const int gcol = col0 + ecol;
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
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(strip + lrow * PITCH + 32 * j + 8 * g + 4 * lhalf) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                  acc[i][j][4 * g + 3]};
#pragma unroll
    for (int pass = 0; pass < 32 / ROWS_PER_PASS; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* src = strip + rr * PITCH + ecol;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_epilogue<EPI>(v[e], bias[e]);
      const int row = row0 + 32 * i + rr;
      if (row < p.M) store_row8<OUT_BF16>(v, row, gcol, full_cols, p);
    }
  }
}

// Epilogue of one wave for the 16 x 16 accumulator layout (element e of
// lane l of block (i, j) is row 16 i + l%16, column 16 j + 4 (l/16) + e):
// each 16-row strip of the wave's tile goes through a private LDS strip so
// that every lane stores 8 consecutive outputs; bias, tanh-GeLU and rounding
// as store_wave_tile.
template <int EPI, bool OUT_BF16, int FM, int FN>
__device__ __forceinline__ void store_wave_tile16(const f32x4 (&acc)[FM][FN], float* strip, int lane,
                                                  int row0, int col0, const Bf16Args& p) {
  constexpr int WTN = 16 * FN;
  constexpr int PITCH = WTN + 4;  // floats; 16 bytes of padding per row
  constexpr int LANES_PER_ROW = WTN / 8;
  constexpr int ROWS_PER_PASS = kWave / LANES_PER_ROW;
  static_assert(16 % ROWS_PER_PASS == 0, "whole passes per strip");
  const int l16 = lane & 15, lq = lane >> 4;
  const int erow = lane / LANES_PER_ROW;
  const int ecol = 8 * (lane % LANES_PER_ROW);
  const int gcol = col0 + ecol;
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
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) *reinterpret_cast<f32x4*>(strip + l16 * PITCH + 16 * j + 4 * lq) = acc[i][j];
#pragma unroll
    for (int pass = 0; pass < 16 / ROWS_PER_PASS; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* src = strip + rr * PITCH + ecol;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_epilogue<EPI>(v[e], bias[e]);
      const int row = row0 + 16 * i + rr;
      if (row < p.M) store_row8<OUT_BF16>(v, row, gcol, full_cols, p);
    }
  }
}

// Quantising epilogue of one wave (DeepGEMM page, section 1.2: activation,
// quantisation and scaling welded into the producing kernel).  Each output
// is epilogue(acc + bias) rounded to bf16, exactly what the plain epilogue
// stores; the values are then quantised in groups of 128 consecutive
// columns of a row, as the standalone 1 x 128 quantiser does (same scale,
// quotient and rounding code), so codes and scales equal that quantiser's on
// the bf16 output, bit for bit.  A 128-column group spans two waves (wave
// tiles are 64 columns wide), so the group maximum goes through LDS:
// phase 1 forms each row's maximum over the wave's 64 columns (8 lanes hold
// a row after the LDS strip transpose) into amax_tab[row][wn], keeping the
// rounded values in registers; after a barrier, phase 2 combines the two
// halves, writes 8 codes (8 bytes) per lane and, from the even wave of the
// pair, the group's scale.  Rows >= M and columns >= N are not stored.
template <int EPI, int FM, int FN, int WN>
__device__ __forceinline__ void store_wave_tile_q8(const f32x16 (&acc)[FM][FN], float* strip,
                                                   float* amax_tab, int lane, int wn, int trow0,
                                                   int row0, int col0, const Bf16Args& p) {
  constexpr int WTN = 32 * FN;
  static_assert(WTN == 64, "a 128-column group must span a wave pair");
  constexpr int PITCH = WTN + 4;
  constexpr int LANES_PER_ROW = WTN / 8;
  constexpr int ROWS_PER_PASS = kWave / LANES_PER_ROW;
  constexpr int PASSES = 32 / ROWS_PER_PASS;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int erow = lane / LANES_PER_ROW;
  const int ecol = 8 * (lane % LANES_PER_ROW);
  const int gcol = col0 + ecol;
  float bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bias[e] = 0.0f;
    if constexpr (EPI != kEpiNone) {
      if (gcol + e < p.N) bias[e] = bf16_bits_to_f32(p.bias[gcol + e]);
    }
  }
  // Phase 1: rounded outputs (packed bf16 pairs) and per-row partial maxima.
  u32x4 hv[FM][PASSES];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(strip + lrow * PITCH + 32 * j + 8 * g + 4 * lhalf) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                  acc[i][j][4 * g + 3]};
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* src = strip + rr * PITCH + ecol;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gcol + e < p.N ? apply_epilogue<EPI>(v[e], bias[e]) : 0.0f;
      const u32x4 h = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
      hv[i][pass] = h;
      float m = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(h[d] << 16)));
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(h[d] & 0xffff0000u)));
      }
#pragma unroll
      for (int d = 1; d < LANES_PER_ROW; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d, kWave));
      if (lane % LANES_PER_ROW == 0) amax_tab[(trow0 + 32 * i + rr) * WN + wn] = m;
    }
  }
  __syncthreads();
  // Phase 2: the pair's maximum, scale, codes.
  const int G = (p.N + 127) / 128;
  uint8_t* const q = static_cast<uint8_t*>(p.C);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* t = amax_tab + (trow0 + 32 * i + rr) * WN;
      const float amax = __builtin_fmaxf(t[wn], t[wn ^ 1]);
      const float scale = fp8q::group_scale(amax);
      const u32x4 h = hv[i][pass];
      float x[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        x[2 * d] = __uint_as_float(h[d] << 16);
        x[2 * d + 1] = __uint_as_float(h[d] & 0xffff0000u);
      }
      const u32x2 codes = fp8q::codes8(x, scale);
      const int row = row0 + 32 * i + rr;
      if (row < p.M) {
        uint8_t* out = q + static_cast<int64_t>(row) * p.ldc + gcol;
        if (p.vec_c && gcol + 8 <= p.N) {
          *reinterpret_cast<u32x2*>(out) = codes;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gcol + e < p.N) out[e] = static_cast<uint8_t>(codes[e / 4] >> (8 * (e % 4)));
        }
        if ((wn & 1) == 0 && ecol == 0 && col0 < p.N)
          p.qscale[static_cast<int64_t>(row) * G + col0 / 128] = scale;
      }
    }
  }
}

// The quantising epilogue for the 16 x 16 accumulator layout (element e of
// lane l of block (i, j) is row 16 i + l%16, column 16 j + 4 (l/16) + e):
// the same two phases, each 16-row strip of the wave's tile going through
// the wave's LDS strip as in store_wave_tile16.
template <int EPI, int FM, int FN, int WN>
__device__ __forceinline__ void store_wave_tile16_q8(const f32x4 (&acc)[FM][FN], float* strip,
                                                     float* amax_tab, int lane, int wn, int trow0,
                                                     int row0, int col0, const Bf16Args& p) {
  constexpr int WTN = 16 * FN;
  static_assert(WTN == 64, "a 128-column group must span a wave pair");
  constexpr int PITCH = WTN + 4;
  constexpr int LANES_PER_ROW = WTN / 8;
  constexpr int ROWS_PER_PASS = kWave / LANES_PER_ROW;
  constexpr int PASSES = 16 / ROWS_PER_PASS;
  const int l16 = lane & 15, lq = lane >> 4;
  const int erow = lane / LANES_PER_ROW;
  const int ecol = 8 * (lane % LANES_PER_ROW);
  const int gcol = col0 + ecol;
  float bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bias[e] = 0.0f;
    if constexpr (EPI != kEpiNone) {
      if (gcol + e < p.N) bias[e] = bf16_bits_to_f32(p.bias[gcol + e]);
    }
  }
  // Phase 1: rounded outputs (packed bf16 pairs) and per-row partial maxima.
  u32x4 hv[FM][PASSES];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) *reinterpret_cast<f32x4*>(strip + l16 * PITCH + 16 * j + 4 * lq) = acc[i][j];
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* src = strip + rr * PITCH + ecol;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gcol + e < p.N ? apply_epilogue<EPI>(v[e], bias[e]) : 0.0f;
      const u32x4 h = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
      hv[i][pass] = h;
      float m = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(h[d] << 16)));
        m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(h[d] & 0xffff0000u)));
      }
#pragma unroll
      for (int d = 1; d < LANES_PER_ROW; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d, kWave));
      if (lane % LANES_PER_ROW == 0) amax_tab[(trow0 + 16 * i + rr) * WN + wn] = m;
    }
  }
  __syncthreads();
  // Phase 2: the pair's maximum, scale, codes.
  const int G = (p.N + 127) / 128;
  uint8_t* const q = static_cast<uint8_t*>(p.C);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int rr = erow + ROWS_PER_PASS * pass;
      const float* t = amax_tab + (trow0 + 16 * i + rr) * WN;
      const float amax = __builtin_fmaxf(t[wn], t[wn ^ 1]);
      const float scale = fp8q::group_scale(amax);
      const u32x4 h = hv[i][pass];
      float x[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        x[2 * d] = __uint_as_float(h[d] << 16);
        x[2 * d + 1] = __uint_as_float(h[d] & 0xffff0000u);
      }
      const u32x2 codes = fp8q::codes8(x, scale);
      const int row = row0 + 16 * i + rr;
      if (row < p.M) {
        uint8_t* out = q + static_cast<int64_t>(row) * p.ldc + gcol;
        if (p.vec_c && gcol + 8 <= p.N) {
          *reinterpret_cast<u32x2*>(out) = codes;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gcol + e < p.N) out[e] = static_cast<uint8_t>(codes[e / 4] >> (8 * (e % 4)));
        }
        if ((wn & 1) == 0 && ecol == 0 && col0 < p.N)
          p.qscale[static_cast<int64_t>(row) * G + col0 / 128] = scale;
      }
    }
  }
}

// Global -> LDS loads of one workgroup's A and B slices, shared by both MFMA
// shapes.  A block i of a wave covers 16-byte slots S = 64*blk + lane; slot
// S is chunk (S % A_CPR) ^ a_swz(row) of row S / A_CPR.  B likewise with
// b_swz.  Every byte offset is carried in the per-lane offset so the buffer
// range check sees all of it; OR-ing in kOutOfRange (offsets stay below
// 2^31) turns a load into zeros.  The windows of the slice at column k0 are
// A rows m0 .. M-1 from column k0 and B rows k0 .. K-1 from column n0 (BT:
// B rows n0 .. N-1 from column k0), so bytes past M, N or K read as zeros;
// the main loops step a pointer and a size by one slice per iteration
// instead of recomputing them.
// WIN, the launcher's choice of windows:
//   kWinSlice -- the windows of each slice, as above, with a per-lane check
//                of the chunk's K columns;
//   kWinWhole -- when every offset of the call stays below 2^31 and K is a
//                multiple of BK: one window per operand covers all of K,
//                built and made uniform once, and the slice's K offset rides
//                in the per-lane offset (building two windows per slice cost
//                4-7 % on the 4096^3 and FFN shapes); a slice lies wholly
//                inside K or wholly past it, so the K check is one uniform
//                compare instead of one per lane (2-3 % more).
constexpr int kWinSlice = 0, kWinWhole = 1;
template <class C, bool BT, int WIN>
struct TileLoader {
  static constexpr bool WHOLE = WIN == kWinWhole;
  uint32_t a_goff[C::APW];
  int a_kc[C::APW];
  uint32_t b_goff[C::BPW];
  int b_kc[C::BPW];  // BT: first K column of the chunk
  const uint16_t* a_base0;
  int64_t a_size0;
  const uint16_t* b_base0;
  int64_t b_size0;
  int64_t b_step;  // elements per slice
  int64_t ldb;
  uint32_t smem_base;
  int wave, K;

  __device__ __forceinline__ TileLoader(const Bf16Args& p, int wave_, int lane, int m0, int n0,
                                        uint32_t smem_base_)
      : ldb(p.ldb), smem_base(smem_base_), wave(wave_), K(p.K) {
    const int64_t lda2 = p.lda * 2, ldb2 = p.ldb * 2;
#pragma unroll
    for (int i = 0; i < C::APW; ++i) {
      const int s = 64 * (wave * C::APW + i) + lane;
      const int r = s / C::A_CPR;
      const int c = (s % C::A_CPR) ^ a_swz<C>(r);
      a_goff[i] = static_cast<uint32_t>(r * lda2 + 16 * c);
      a_kc[i] = 8 * c;
    }
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      const int s = 64 * (wave * C::BPW + i) + lane;
      if constexpr (BT) {
        const int n = s / C::A_CPR;
        const int c = (s % C::A_CPR) ^ a_swz<C>(n);
        b_goff[i] = static_cast<uint32_t>(n * ldb2 + 16 * c);
        b_kc[i] = 8 * c;
      } else {
        const int k = s / C::B_CPR;
        const int c = (s % C::B_CPR) ^ b_swz<C>(k);
        b_goff[i] = static_cast<uint32_t>(k * ldb2 + 16 * c) | (n0 + 8 * c < p.N ? 0u : kOutOfRange);
        b_kc[i] = 0;
      }
    }
    a_base0 = p.A + static_cast<int64_t>(m0) * p.lda;
    a_size0 = (static_cast<int64_t>(p.M - m0 - 1) * p.lda + p.K) * 2;
    b_base0 = BT ? p.B + static_cast<int64_t>(n0) * p.ldb : p.B + n0;
    b_size0 = BT ? (static_cast<int64_t>(p.N - n0 - 1) * p.ldb + p.K) * 2
                 : (static_cast<int64_t>(p.K - 1) * p.ldb + (p.N - n0)) * 2;
    b_step = BT ? int64_t{C::BK} : static_cast<int64_t>(C::BK) * p.ldb;
    if constexpr (WHOLE) {
      wa_all = uniform_words(make_window_words(a_base0, a_size0));
      wb_all = uniform_words(make_window_words(b_base0, b_size0));
    }
  }
  i32x4 wa_all, wb_all;  // WHOLE: the operands' windows over all of K
  __device__ __forceinline__ i32x4 window_a(int k0) const {
    if constexpr (WHOLE) return wa_all;
    else return make_window_words(a_base0 + k0, a_size0 - 2 * k0);
  }
  __device__ __forceinline__ i32x4 window_b(int k0) const {
    if constexpr (WHOLE) return wb_all;
    const int64_t e = BT ? int64_t{k0} : static_cast<int64_t>(k0) * ldb;
    return make_window_words(b_base0 + e, b_size0 - 2 * e);
  }
  __device__ __forceinline__ void issue_a(i32x4 w, int stage, int k0, int i) const {
    const uint32_t lds = smem_base + stage * C::STAGE + (wave * C::APW + i) * 1024;
    const uint32_t oor = (WHOLE ? k0 < K : k0 + a_kc[i] < K) ? 0u : kOutOfRange;
    if constexpr (WHOLE) buf_load16_lds_u(w, lds, (a_goff[i] + 2u * static_cast<uint32_t>(k0)) | oor);
    else buf_load16_lds(w, lds, a_goff[i] | oor);
  }
  __device__ __forceinline__ void issue_b(i32x4 w, int stage, int k0, int i) const {
    const uint32_t lds = smem_base + stage * C::STAGE + C::A_STAGE + (wave * C::BPW + i) * 1024;
    const uint32_t oor = BT && (WHOLE ? k0 >= K : k0 + b_kc[i] >= K) ? kOutOfRange : 0u;
    // [K, N]: a column past N keeps its out-of-range bit through the add
    // (the sum stays below 2^32).
    const uint32_t koff = 2u * static_cast<uint32_t>(k0) * (BT ? 1u : static_cast<uint32_t>(ldb));
    if constexpr (WHOLE) buf_load16_lds_u(w, lds, (b_goff[i] + koff) | oor);
    else buf_load16_lds(w, lds, b_goff[i] | oor);
  }
  // Slices 0 .. NS-2 into stages 0 .. NS-2 (past K the loads read zeros).
  __device__ __forceinline__ void prologue() const {
    static_for<C::NS - 1>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const i32x4 wa = window_a(s * C::BK), wb = window_b(s * C::BK);
#pragma unroll
      for (int i = 0; i < C::APW; ++i) issue_a(wa, s, s * C::BK, i);
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) issue_b(wb, s, s * C::BK, i);
    });
  }
};

template <class C, bool BT, int EPI, bool OUT_BF16, bool QUANT, int WIN>
__global__ __launch_bounds__(C::THREADS, 1) void tgemm_bf16_tiled(Bf16Args p, int tiles_m,
                                                                int tiles_n) {
  static_assert(C::MF == 32, "the 32 x 32 x 16 kernel");
  apply_batch(p, OUT_BF16 ? 2 : 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS load bases)
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  // acc[i][j] holds the transposed 32 x 32 block (MFMA operands swapped):
  // element 4*g + e of lane l is row 32*i + l%32, column 32*j + 8*g + 4*(l/32) + e.
  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

  // ---- global -> LDS ----
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  const TileLoader<C, BT, WIN> ld(p, wave, lane, m0, n0, smem_base);

  // ---- LDS -> registers ----
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  // A operand of block i, sub-step ks: row wm*WTM + 32i + lrow, chunk 2ks + lhalf.
  // The swizzle depends only on lrow (32i and wm*WTM are multiples of 16).
  const int a_rd = (wm * C::WTM + lrow) * C::A_ROW;
  const int a_x = a_swz<C>(lrow);
  // B operand of block j: transposed reads; lane L = 16g + 4e + q supplies
  // K row 8(g>>1) + e (+4 for the second half) and columns 16(g&1) + 4q .. +3
  // of the block, and receives 4 k of column 16(g&1) + (L%16).
  const int bg = lane >> 4, be = (lane >> 2) & 3, bq = lane & 3;
  // BT: B operand of block j, sub-step ks: row wn*WTN + 32j + lrow of the
  // K-contiguous tile, chunk 2ks + lhalf, as for A.
  int b_rd[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    if constexpr (BT) {
      b_rd[j] = C::A_STAGE + (wn * C::WTN + 32 * j + lrow) * C::A_ROW;
    } else {
      const int chunk = (((wn * C::WTN / 32) + j) ^ be) * 4 + 2 * (bg & 1) + (bq >> 1);
      b_rd[j] = C::A_STAGE + (8 * (bg >> 1) + be) * C::B_ROW + chunk * 16 + 8 * (bq & 1);
    }
  }
  constexpr int kNR = C::FM + C::FN;
  bf16x8 fa[2][C::FM], fb[2][C::FN];
  // Fragment f < FM is A block f, the rest are B blocks.
  auto lds_read = [&](int buf, int stage, int ks, int f) {
    const uint8_t* base = smem + stage * C::STAGE;
    if (f < C::FM) {
      const int off = a_rd + 32 * f * C::A_ROW + (((2 * ks + lhalf) ^ a_x) * 16);
      fa[buf][f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
    } else if constexpr (BT) {
      const int off = b_rd[f - C::FM] + (((2 * ks + lhalf) ^ a_x) * 16);
      fb[buf][f - C::FM] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
    } else {
      const int j = f - C::FM;
      const uint8_t* q = base + b_rd[j] + 16 * ks * C::B_ROW;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, q));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, q + 4 * C::B_ROW));
      fb[buf][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  constexpr int kQ = C::FM * C::FN;
  auto mfma_one = [&](int buf, int q) {
    const int i = q / C::FN, j = q % C::FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };

  // Slot schedule of slice t (stage t % NS holds it; the loads of slice
  // t+NS-1 go to the stage slice t-1 occupied).  Slots 0 .. KS*kQ-1 are the
  // slice's MFMAs, sub-step u = slot / kQ using operand buffer u & 1:
  //   loads of slice t+NS-1           spread over [0, kLoadEnd), at most one
  //                                   per slot, so the vector memory path is
  //                                   not flooded in bursts
  //   operands of sub-step u+1        [u*kQ, u*kQ + kQ/2)   (u < KS-1)
  //   wait for slice t+1, barrier     before slot kBar
  //   operands of sub-step 0, t+1     [kBar, kBar + kQ/4)
  // The barrier also certifies that every wave has finished reading the
  // stage the next iteration's loads overwrite.
  constexpr int kSlots = C::KS * kQ;
  constexpr int kBar = (C::NS == 2) ? kSlots - kQ / 2 : (C::KS - 1) * kQ;
  // With two stages slice t+1 is loaded in this very iteration, so all of
  // its loads must precede the barrier.
  constexpr int kLoadEnd = (C::NS == 2) ? (kBar < kSlots / C::SPREAD ? kBar : kSlots / C::SPREAD)
                                       : kSlots / C::SPREAD;
  static_assert(kLoadEnd >= C::LPS || C::LPS > kSlots, "one load per slot");
  auto load_slot = [](int l) { return spread(l, C::LPS, 0, kLoadEnd); };
  // Loads younger than slice t+1 when the barrier waits: the NS-3 slices
  // issued in earlier iterations after it, plus this iteration's loads
  // issued before the barrier.
  constexpr int kBefore = [] {
    int n = 0;
    for (int l = 0; l < C::LPS; ++l) n += (spread(l, C::LPS, 0, kLoadEnd) < kBar) ? 1 : 0;
    return n;
  }();
  constexpr int kAhead = (C::NS == 2) ? 0 : (C::NS - 3) * C::LPS + kBefore;
  static_assert(kBar + kQ / 4 <= kSlots, "slot schedule");

  const int KT = (p.K + C::BK - 1) / C::BK;
  if (KT > 0) {
    ld.prologue();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::NS - 2) * C::LPS) : "memory");
    lds_barrier();
#pragma unroll
    for (int f = 0; f < kNR; ++f) lds_read(0, 0, 0, f);

    int cur = 0;
    int lst = C::NS - 1;  // stage receiving slice t+NS-1
    // Windows of slice t+NS-1, stepped once per iteration.
    const uint16_t* a_ptr = ld.a_base0 + (C::NS - 1) * C::BK;
    int64_t a_left = ld.a_size0 - 2 * (C::NS - 1) * C::BK;
    const uint16_t* b_ptr = ld.b_base0 + (C::NS - 1) * ld.b_step;
    int64_t b_left = ld.b_size0 - 2 * (C::NS - 1) * ld.b_step;
    for (int t = 0; t < KT; ++t) {
      const int nxt = cur + 1 == C::NS ? 0 : cur + 1;
      const int kl = (t + C::NS - 1) * C::BK;
      i32x4 wa, wb;
      if constexpr (WIN == kWinWhole) {
        wa = ld.wa_all;
        wb = ld.wb_all;
      } else {
        wa = make_window_words(a_ptr, a_left);
        wb = make_window_words(b_ptr, b_left);
        a_ptr += C::BK;
        a_left -= 2 * C::BK;
        b_ptr += ld.b_step;
        b_left -= 2 * ld.b_step;
      }
      static_for<kSlots>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int u = s / kQ;
        if constexpr (s == kBar) {
          TGEMM_SCHED_FENCE();
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAhead) : "memory");
          lds_barrier();
        }
        TGEMM_SCHED_FENCE();
        mfma_one(u & 1, s % kQ);
        TGEMM_SCHED_FENCE();
        static_for<kNR>([&](auto fc) {
          constexpr int f = decltype(fc)::value;
          if constexpr (u + 1 < C::KS && spread(f, kNR, u * kQ, u * kQ + kQ / 2) == s)
            lds_read((u + 1) & 1, cur, u + 1, f);
          if constexpr (spread(f, kNR, kBar, kBar + kQ / 4) == s) lds_read(0, nxt, 0, f);
        });
        static_for<C::APW>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (load_slot(i) == s) ld.issue_a(wa, lst, kl, i);
        });
        static_for<C::BPW>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (load_slot(C::APW + i) == s) ld.issue_b(wb, lst, kl, i);
        });
      });
      TGEMM_SCHED_FENCE();
      lst = cur;
      cur = nxt;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
  lds_barrier();  // every wave is done with the operand stages

  // ---- epilogue ----
  if constexpr (QUANT) {
    static_assert((C::WAVES * 32 * C::EPI_PITCH + C::BM * C::WN) * 4 <= C::LDS_BYTES,
                  "strips and the row-maximum table must fit in LDS");
    store_wave_tile_q8<EPI, C::FM, C::FN, C::WN>(
        acc, reinterpret_cast<float*>(smem) + wave * 32 * C::EPI_PITCH,
        reinterpret_cast<float*>(smem) + C::WAVES * 32 * C::EPI_PITCH, lane, wn, wm * C::WTM,
        m0 + wm * C::WTM, n0 + wn * C::WTN, p);
  } else {
    store_wave_tile<EPI, OUT_BF16, C::FM, C::FN>(
        acc, reinterpret_cast<float*>(smem) + wave * 32 * C::EPI_PITCH, lane, m0 + wm * C::WTM,
        n0 + wn * C::WTN, p);
  }
}


// The same GEMM with v_mfma_f32_16x16x32_bf16.  On random data the matrix
// units deliver more FLOP per watt with this shape than with 32 x 32 x 16
// (an MFMA-only loop on N(0,1)-like bf16 operands: 1.90 against 1.69
// PFLOP/s on MI355X, whose bf16 GEMMs run power-bound), for the same LDS
// traffic: a wave's operands per 32-wide slice are still its WTM rows of A
// and WTN columns of B.  A slice is one MFMA step, so the schedule differs:
//   * per slice, slot s runs the MFMA of block (s / FN, s % FN) (row-major);
//   * the barrier sits before slot BAR and certifies that slice t+1 has
//     landed; every operand read of slice t+1 comes after it;
//   * an A operand is single-buffered: after the last MFMA of row block i
//     (or right after the barrier, if that comes later) the next slice's row
//     block i is read into the same registers;
//   * B operands are double-buffered by slice parity (the loop is unrolled
//     by two): the next slice's are read in the half slice after the barrier;
//   * the loads of slice t+NS-1 are spread over the slots; they refill the
//     stage of slice t-1, whose last reads came before the previous barrier.
// Operand layouts (16 x 16 x 32): an A operand gives lane l row l%16 of its
// block and K 8(l/16) .. +7 of the slice (one 16-byte read); a B operand
// gives lane l column l%16 and the same K (two transposed reads: lane
// 16g + 4e + q supplies K rows 8g + e and 8g + 4 + e, columns 4q .. 4q+3).
// The operands are swapped as in the 32 x 32 kernel, so element e of lane l
// of block (i, j) is row 16 i + l%16, column 16 j + 4 (l/16) + e.
template <class C, bool BT, int EPI, bool OUT_BF16, bool QUANT, int WIN>
__global__ __launch_bounds__(C::THREADS, 1) void tgemm_bf16_tiled16(Bf16Args p, int tiles_m,
                                                                  int tiles_n) {
  static_assert(C::MF == 16 && C::KS == 1, "one 16 x 16 x 32 step per slice");
  static_assert(C::NS >= 3, "the slice after next is in flight at each barrier");
  apply_batch(p, OUT_BF16 ? 2 : 4);
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN;
  const int wn = wave % C::WN;

  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * C::BM;
  const int n0 = tn * C::BN;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{};

  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  const TileLoader<C, BT, WIN> ld(p, wave, lane, m0, n0, smem_base);

  // ---- LDS -> registers ----
  const int l16 = lane & 15, lq = lane >> 4;
  // A row block i: row wm*WTM + 16i + l16, chunk lq (the swizzle depends on
  // l16 only: 16i and wm*WTM are multiples of 16).
  const int a_rd = (wm * C::WTM + l16) * C::A_ROW;
  const int a_ch = ((lq ^ a_swz<C>(l16)) * 16);
  const int bg = lane >> 4, be = (lane >> 2) & 3, bq = lane & 3;
  int b_rd[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    if constexpr (BT) {
      b_rd[j] = C::A_STAGE + (wn * C::WTN + 16 * j + l16) * C::A_ROW + a_ch;
    } else {
      const int k = 8 * bg + be;
      const int chunk = (2 * (wn * C::WTN / 16 + j) + (bq >> 1)) ^ b_swz<C>(k);
      b_rd[j] = C::A_STAGE + k * C::B_ROW + chunk * 16 + 8 * (bq & 1);
    }
  }
  bf16x8 fa[C::FM], fb[2][C::FN];
  auto read_a = [&](int stage, int i) {
    const uint8_t* base = smem + stage * C::STAGE + a_rd + 16 * i * C::A_ROW + a_ch;
    fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base));
  };
  auto read_b = [&](int buf, int stage, int j) {
    const uint8_t* q = smem + stage * C::STAGE + b_rd[j];
    if constexpr (BT) {
      fb[buf][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q));
    } else {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, q));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TGEMM_LDS(i16x4, q + 4 * C::B_ROW));
      fb[buf][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  constexpr int kSlots = C::FM * C::FN;
  constexpr int kBar = C::BAR;
  static_assert(kSlots >= C::LPS && kBar + kSlots / 2 <= kSlots && kBar + C::FM <= kSlots, "slot schedule");
  auto load_slot = [](int l) { return spread(l, C::LPS, 0, kSlots); };
  auto b_slot = [](int j) { return spread(j, C::FN, kBar, kBar + kSlots / 2); };
  auto a_slot = [](int i) { return i * C::FN + C::FN - 1 > kBar + i ? i * C::FN + C::FN - 1 : kBar + i; };
  // Loads younger than slice t+1 when the barrier waits: the NS-3 slices
  // issued in earlier iterations after it, plus this slice's loads issued
  // before the barrier.
  constexpr int kBefore = [] {
    int n = 0;
    for (int l = 0; l < C::LPS; ++l) n += (spread(l, C::LPS, 0, kSlots) < kBar) ? 1 : 0;
    return n;
  }();
  constexpr int kAhead = (C::NS - 3) * C::LPS + kBefore;

  const int KT = (p.K + C::BK - 1) / C::BK;
  if (KT > 0) {
    ld.prologue();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::NS - 2) * C::LPS) : "memory");
    lds_barrier();
#pragma unroll
    for (int i = 0; i < C::FM; ++i) read_a(0, i);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) read_b(0, 0, j);

    int cur = 0;
    int lst = C::NS - 1;  // stage receiving slice t+NS-1
    const uint16_t* a_ptr = ld.a_base0 + (C::NS - 1) * C::BK;
    int64_t a_left = ld.a_size0 - 2 * (C::NS - 1) * C::BK;
    const uint16_t* b_ptr = ld.b_base0 + (C::NS - 1) * ld.b_step;
    int64_t b_left = ld.b_size0 - 2 * (C::NS - 1) * ld.b_step;

    // One slice; P: the B operand buffer holding this slice's operands.
    auto slice = [&](auto pc, int t) {
      constexpr int P = decltype(pc)::value;
      const int nxt = cur + 1 == C::NS ? 0 : cur + 1;
      const int kl = (t + C::NS - 1) * C::BK;
      i32x4 wa, wb;
      if constexpr (WIN == kWinWhole) {
        wa = ld.wa_all;
        wb = ld.wb_all;
      } else {
        wa = make_window_words(a_ptr, a_left);
        wb = make_window_words(b_ptr, b_left);
        a_ptr += C::BK;
        a_left -= 2 * C::BK;
        b_ptr += ld.b_step;
        b_left -= 2 * ld.b_step;
      }
      static_for<kSlots>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int i = s / C::FN, j = s % C::FN;
        if constexpr (s == kBar) {
          TGEMM_SCHED_FENCE();
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAhead) : "memory");
          lds_barrier();
        }
        TGEMM_SCHED_FENCE();
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[P][j], fa[i], acc[i][j], 0, 0, 0);
        TGEMM_SCHED_FENCE();
        static_for<C::FM>([&](auto ic) {
          constexpr int ii = decltype(ic)::value;
          if constexpr (a_slot(ii) == s) read_a(nxt, ii);
        });
        static_for<C::FN>([&](auto jc) {
          constexpr int jj = decltype(jc)::value;
          if constexpr (b_slot(jj) == s) read_b(1 - P, nxt, jj);
        });
        static_for<C::APW>([&](auto ic) {
          constexpr int l = decltype(ic)::value;
          if constexpr (load_slot(l) == s) ld.issue_a(wa, lst, kl, l);
        });
        static_for<C::BPW>([&](auto ic) {
          constexpr int l = decltype(ic)::value;
          if constexpr (load_slot(C::APW + l) == s) ld.issue_b(wb, lst, kl, l);
        });
      });
      TGEMM_SCHED_FENCE();
      lst = cur;
      cur = nxt;
    };
    int t = 0;
    for (; t + 1 < KT; t += 2) {
      slice(std::integral_constant<int, 0>{}, t);
      slice(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < KT) slice(std::integral_constant<int, 0>{}, t);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
  lds_barrier();  // every wave is done with the operand stages

  static_assert(C::WAVES * 16 * (C::WTN + 4) * 4 <= C::LDS_BYTES, "epilogue strips fit in LDS");
  if constexpr (QUANT) {
    static_assert((C::WAVES * 16 * (C::WTN + 4) + C::BM * C::WN) * 4 <= C::LDS_BYTES,
                  "strips and the row-maximum table must fit in LDS");
    store_wave_tile16_q8<EPI, C::FM, C::FN, C::WN>(
        acc, reinterpret_cast<float*>(smem) + wave * 16 * (C::WTN + 4),
        reinterpret_cast<float*>(smem) + C::WAVES * 16 * (C::WTN + 4), lane, wn, wm * C::WTM, m0 + wm * C::WTM,
        n0 + wn * C::WTN, p);
  } else {
    store_wave_tile16<EPI, OUT_BF16, C::FM, C::FN>(acc, reinterpret_cast<float*>(smem) + wave * 16 * (C::WTN + 4),
                                                   lane, m0 + wm * C::WTM, n0 + wn * C::WTN, p);
  }
}

// Whole-K windows fit when every per-lane offset of the call stays below
// 2^31: a tile's rows of A plus K, and B's rows (all of K for [K, N], a
// tile's for [N, K]), counting the slices the pipeline loads past K.
template <class C, bool BT>
bool whole_windows_ok(const Bf16Args& a) {
  const int64_t kspan = int64_t{a.K} + int64_t{C::NS + 1} * C::BK;
  const int64_t a_max = (int64_t{C::BM} * a.lda + kspan) * 2;
  const int64_t b_max = BT ? (int64_t{C::BN} * a.ldb + kspan) * 2 : (kspan * a.ldb + C::BN) * 2;
  return a_max < (int64_t{1} << 31) && b_max < (int64_t{1} << 31);
}

template <class C, bool BT, int EPI, bool OUT_BF16, bool QUANT, int WIN>
hipError_t launch_cw(const Bf16Args& a, hipStream_t s) {
  const int tiles_m = (a.M + C::BM - 1) / C::BM;
  const int tiles_n = (a.N + C::BN - 1) / C::BN;
  if constexpr (C::MF == 16) {
    hipLaunchKernelGGL((tgemm_bf16_tiled16<C, BT, EPI, OUT_BF16, QUANT, WIN>), dim3(tiles_m * tiles_n, a.batch),
                       dim3(C::THREADS), 0, s, a, tiles_m, tiles_n);
  } else {
    hipLaunchKernelGGL((tgemm_bf16_tiled<C, BT, EPI, OUT_BF16, QUANT, WIN>), dim3(tiles_m * tiles_n, a.batch),
                       dim3(C::THREADS), 0, s, a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

template <class C, bool BT, int EPI, bool OUT_BF16, bool QUANT = false>
hipError_t launch_c(const Bf16Args& a, hipStream_t s) {
  if (whole_windows_ok<C, BT>(a) && a.K % C::BK == 0) return launch_cw<C, BT, EPI, OUT_BF16, QUANT, kWinWhole>(a, s);
  return launch_cw<C, BT, EPI, OUT_BF16, QUANT, kWinSlice>(a, s);
}

template <class C>
hipError_t dispatch_q8(const Bf16Args& a, int epi, hipStream_t s) {
  if (epi == kEpiNone) return launch_c<C, false, kEpiNone, true, true>(a, s);
  if (epi == kEpiBias) return launch_c<C, false, kEpiBias, true, true>(a, s);
  return launch_c<C, false, kEpiBiasGelu, true, true>(a, s);
}

template <class C, bool BT>
hipError_t dispatch_epi(const Bf16Args& a, int epi, int out_bf16, hipStream_t s) {
  if (out_bf16) {
    if (epi == kEpiNone) return launch_c<C, BT, kEpiNone, true>(a, s);
    if (epi == kEpiBias) return launch_c<C, BT, kEpiBias, true>(a, s);
    return launch_c<C, BT, kEpiBiasGelu, true>(a, s);
  }
  if (epi == kEpiNone) return launch_c<C, BT, kEpiNone, false>(a, s);
  if (epi == kEpiBias) return launch_c<C, BT, kEpiBias, false>(a, s);
  return launch_c<C, BT, kEpiBiasGelu, false>(a, s);
}

// Per tile shape (measured on MI355X): BK = 32 keeps several slices of
// loads in flight (five stages on 256 x 256, four on 128 x 128); the
// 256 x 256 tile runs 8 waves (two per SIMD, each 128 x 64 outputs), which
// hides one wave's LDS and memory waits behind the other's MFMAs, with the
// 16 x 16 x 32 MFMA (2-3 % faster than 32 x 32 x 16 there, bit-identical
// results; on the 256 x 128 tile it measured 10-50 % slower, so that tile
// keeps 32 x 32 x 16 with 64-wide slices).
using Cfg256x256 = Cfg<256, 256, 32, 5, 1, 4, 16, 16>;
using Cfg256x128 = Cfg<256, 128, 64, 3>;
// The quantising epilogue on the 256 x 256 tile uses the same 16 x 16 kernel.
using Cfg256x256Q = Cfg256x256;
using Cfg256x128Q = Cfg<256, 128, 64, 3>;
using Cfg128x128 = Cfg<128, 128, 64, 4>;

}  // namespace

TiledShapeInfo tiled_shape_info(int shape) {
  switch (shape) {
    case kTile256x256: return {256, 256, "tgemm_bf16_tiled_256x256x32"};
    case kTile256x128: return {256, 128, "tgemm_bf16_tiled_256x128x64"};
    default: return {128, 128, "tgemm_bf16_tiled_128x128x64"};
  }
}

bool bf16_direct_ok(const Bf16Args& a, int shape) {
  const TiledShapeInfo info = tiled_shape_info(shape);
  // Largest per-lane offsets: a tile's rows of A, a slice's rows of B.
  return a.vec_a && a.vec_b && a.K % 8 == 0 && a.N % 8 == 0 &&
         a.lda * 2 * info.bm < (int64_t{1} << 31) && a.ldb * 2 * 64 < (int64_t{1} << 31);
}

bool bf16_bt_direct_ok(const Bf16Args& a, int shape) {
  const TiledShapeInfo info = tiled_shape_info(shape);
  // Largest per-lane offsets: a tile's rows of A and of B.
  return a.vec_a && a.vec_b && a.K % 8 == 0 && a.lda * 2 * info.bm < (int64_t{1} << 31) &&
         a.ldb * 2 * info.bn < (int64_t{1} << 31);
}

hipError_t launch_bf16_tiled(const Bf16Args& a, int shape, int epi, int out_bf16,
                             hipStream_t s) {
  if (!bf16_direct_ok(a, shape)) return launch_bf16_general(a, shape, epi, out_bf16, s);
  switch (shape) {
    case kTile256x256: return dispatch_epi<Cfg256x256, false>(a, epi, out_bf16, s);
    case kTile256x128: return dispatch_epi<Cfg256x128, false>(a, epi, out_bf16, s);
    default: return dispatch_epi<Cfg128x128, false>(a, epi, out_bf16, s);
  }
}

hipError_t launch_bf16_tiled_q8(const Bf16Args& a, int shape, int epi, hipStream_t s) {
  if (!bf16_direct_ok(a, shape) || a.batch != 1 || a.qscale == nullptr) return hipErrorInvalidValue;
  switch (shape) {
    case kTile256x256: return dispatch_q8<Cfg256x256Q>(a, epi, s);
    case kTile256x128: return dispatch_q8<Cfg256x128Q>(a, epi, s);
    default: return dispatch_q8<Cfg128x128>(a, epi, s);
  }
}

hipError_t launch_bf16_tiled_bt(const Bf16Args& a, int shape, int epi, int out_bf16,
                                hipStream_t s) {
  if (!bf16_bt_direct_ok(a, shape)) return hipErrorInvalidValue;
  switch (shape) {
    case kTile256x256: return dispatch_epi<Cfg256x256, true>(a, epi, out_bf16, s);
    case kTile256x128: return dispatch_epi<Cfg256x128, true>(a, epi, out_bf16, s);
    default: return dispatch_epi<Cfg128x128, true>(a, epi, out_bf16, s);
  }
}

}  // namespace tgemm
