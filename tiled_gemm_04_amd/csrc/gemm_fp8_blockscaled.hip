// FP8 (OCP e4m3fn) GEMM with per-group fp32 scales for gfx950.
//
//   C[i, j] = sum_g sA[i, g] * sB[g, j / 128] * sum_{k in group g} A[i, k] * B[k, j]
//
// DeepGEMM page, section 2.4: low-precision inputs carry a scale per row
// group or small block (here 1 x 128 along K for A, 128 x 128 for B), the
// products are accumulated in fp32, and the scales bring the sum back to the
// output format (bf16).
//
// Mapping onto CDNA4:
//   * one K slice is exactly one scale group (128 bytes of K), and one
//     v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 exponents 127 = 2^0)
//     computes a 16 x 16 block's exact partial sum of the group into a
//     short-lived temporary; one FMA per element folds it into the fp32
//     accumulator: acc += P_g * (sA[i, g] * sB[g, J]).  The E8M0 block
//     exponents of the instruction cannot hold arbitrary fp32 scales, hence
//     the FMA (a 64-byte slice would need it twice per group);
//   * the MFMA operands are swapped (B as the first operand) so each lane's
//     accumulators belong to one output row: the row scale sA is one value
//     per lane and 16-row block, and the column scale sB one value per wave
//     (a wave's 64 columns lie inside one 128-column scale block);
//   * the accumulators are updated by vector FMAs, so they live in
//     architectural VGPRs; two waves per SIMD (8 waves, 512 threads) give
//     each wave 256 of them, and each wave owns a 128 x 64 block of a
//     256 x 256 tile (128 accumulator registers);
//   * A, B and the tile's column of A-scales go global -> LDS with direct
//     buffer loads (no register staging); B stays N-contiguous in LDS and the
//     K-contiguous B operand is read with ds_read_b64_tr_b8 (within each 16
//     lanes, lane 2e+h supplies 8 columns of K row e and lane i receives
//     column i of the 8 rows), four reads per 32-byte operand; 16-byte chunks
//     of every LDS row are XOR-permuted by the row index so operand reads
//     touch distinct LDS banks;
//   * two LDS stages, and a fixed slot schedule per slice (one MFMA per
//     slot, 8 rows x 4 columns of 16 x 16 blocks): the A operand of row i+1
//     is read during row i; the FMAs of row i run between the MFMAs of row
//     i+1 (those of the last row at the start of the next slice), so no FMA
//     waits on a fresh MFMA result; the barrier sits before the last row,
//     whose operands are already in registers, and the next slice's B
//     operands replace the current ones one by one behind its MFMAs; the
//     loads of slice g+2 start right after that barrier (every wave is done
//     with the stage) and finish early in slice g+1, one per slot.
//
// Tile scheduler (DeepGEMM page, section 2.1: a grid too small for the
// machine leaves compute units idle).  Without a workspace, a last round of
// tiles that would occupy at most half of the compute units (one workgroup
// per unit) runs as two 128-row halves per tile, each over all of K: the
// same MFMAs and folds per output element, so the result is bit-identical,
// with twice as many units at work.  With a caller workspace, when the
// tiles would keep at most a quarter of the units busy, each tile is split
// along K instead into P parts of whole scale groups, P = min(CUs / tiles,
// groups / 8, 8); a caller may also force a split of the last round of a
// longer grid.  Every part writes its fp32 partial tile to the workspace
// and bumps a per-tile counter there; the part that arrives last adds the
// partials in part order (the same sum whatever the arrival order), resets
// the counter and runs the epilogue.  No workgroup ever waits for another.
//
// Requirements (checked by the launcher, otherwise the general kernel runs):
// K a multiple of 16 (whole 16-byte chunks of A along K) and per-lane byte
// offsets below 2^31.  Rows of A, B and C need no particular alignment: the
// 16-byte buffer loads are byte-addressed (gfx9 unaligned access mode; on
// MI355X they return the exact bytes at any offset), B columns past N only
// reach accumulators of columns that are never stored, and the stores use
// unaligned 16-byte writes when C rows are not 16-byte aligned.
#include "common.h"
#include "launch.h"

namespace tgemm {

namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;  // bytes of K per slice == one scale group
constexpr int kWTN = 64;   // wave tile columns: 2 (M) x 4 (N) waves
constexpr int kFN = kWTN / 16;
constexpr int kBStage = kBK * kBN;
constexpr int kBBlocks = kBStage / 1024 / 4;  // 1 KiB direct B loads per B wave (4-7) and slice
constexpr int kGroupM = 4;
constexpr int kScaleOne = 127;  // E8M0 exponent of 1.0
constexpr int kFmtE4M3 = 0;     // f8f6f4 operand format code for FP8 E4M3
constexpr int kEpiPitch = kWTN + 4;  // floats per row of the epilogue strip
// s_waitcnt immediate for vmcnt(0) with the other counters unconstrained
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;
static_assert(128 % kWTN == 0, "a wave's columns must sit inside one 128-column scale block");
constexpr int kEarly = 4;  // loads of slice g+2 issued after the barrier of slice g

// Per tile height: a whole tile of kBM = 256 rows, or one of the two 128-row
// halves a tail tile is cut into (see SplitTail).  The waves stay 2 (M) x 4
// (N), each owning kWTM x 64 outputs; waves 0-3 load A (kABlocks blocks of
// 1 KiB per slice), waves 4-7 load B (kBBlocks).  Slot schedule of one slice:
// slot s runs MFMA (s / kFN, s % kFN).
template <int BM>
struct Fp8Shape {
  static constexpr int kBM = BM;
  static constexpr int kWTM = BM / 2;
  static constexpr int kFM = kWTM / 16;
  static constexpr int kAStage = BM * kBK;
  static constexpr int kStage = kAStage + kBStage;
  static constexpr int kABlocks = kAStage / 1024 / 4;
  static constexpr int kSlots = kFM * kFN;
  static constexpr int kBar = kSlots - kFN;  // barrier before the last row
  static_assert(kBar + kEarly <= kSlots && kBBlocks - kEarly <= kBar && kABlocks >= kEarly &&
                    kABlocks <= kBBlocks,
                "load slots");
};
using Fp8Whole = Fp8Shape<kBM>;

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Chunk permutations (physical chunk = logical chunk ^ swizzle(row)).
// A rows are 128 bytes (8 chunks).  An A operand read has lane 16q + r take
// chunks 2q and 2q+1 of row r (r < 16).  Measured with SQ_LDS_BANK_CONFLICT
// on gfx950, r & 7 flipped by bit 3 of r serves all four lane groups without
// conflicts; the plainer (r >> 1) & 7, though it puts each 16-lane group on
// 16 distinct 16-byte bank slots, costs a second cycle on half of the reads.
// The permutation depends on r mod 16 only, so row blocks 16 apart share it.
// B rows are 256 bytes (16 chunks): the 16 K rows k0+e and k0+32+e (e < 8)
// read together by one transposed read land in 16 bank groups.
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int b_swz(int k) { return (k & 7) | (((k >> 5) & 1) << 3); }

// Value of an OCP FP8 E4M3 (e4m3fn) byte: sign, 4 exponent bits with bias
// 7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6), and
// S.1111.111 is NaN (the format has no infinities).
__device__ __forceinline__ float e4m3_value(uint8_t b) {
  const uint32_t em = b & 0x7fu;
  float v;
  if (em == 0x7fu)
    v = __builtin_nanf("");
  else if (em < 8u)
    v = static_cast<float>(em) * 0x1p-9f;
  else
    v = __builtin_bit_cast(float, (((em >> 3) + 120u) << 23) | ((em & 7u) << 20));
  return (b & 0x80u) ? -v : v;
}

// 4-byte buffer load written straight into LDS (lane l -> lds_base + 4 l).
__device__ __forceinline__ void buf_load4_lds(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_words(window))
               : "memory", "m0");
}
// The same for a descriptor already made uniform (as buf_load16_lds_u).
__device__ __forceinline__ void buf_load4_lds_u(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(window)
               : "memory", "m0");
}

// Stores a wave's kFMxkFN blocks of 16 x 16 accumulators (rows row0 + 16 i
// + l%16, columns col0 + 16 j + 4 (l/16) + e) as bf16, through a 16-row
// strip of LDS per wave so that each lane writes 8 consecutive columns.
template <int FM>
__device__ __forceinline__ void store_wave(const f32x4 (&acc)[FM][kFN], float* strip, int lane,
                                           int row0, int col0, const Fp8Args& p) {
  const int l16 = lane & 15, lq = lane >> 4;
  const int erow = lane >> 3;       // 8 rows per pass
  const int ecol = 8 * (lane & 7);  // 8 columns per lane
  const int gcol = col0 + ecol;
  const bool full_cols = p.vec_c && gcol + 8 <= p.N;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < kFN; ++j)
      *reinterpret_cast<f32x4*>(strip + l16 * kEpiPitch + 16 * j + 4 * lq) = acc[i][j];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int rr = erow + 8 * pass;
      const float* src = strip + rr * kEpiPitch + ecol;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      const int row = row0 + 16 * i + rr;
      if (row < p.M) {
        uint16_t* out = p.C + static_cast<int64_t>(row) * p.N + gcol;
        if (full_cols) {
          // Written once, not read back: a non-temporal store.
          __builtin_nontemporal_store(u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                            pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])},
                                      reinterpret_cast<u32x4*>(out));
        } else if (gcol + 8 <= p.N) {
          // Row not 16-byte aligned (N % 8 != 0): one unaligned 16-byte store.
          *reinterpret_cast<u32x4_a2*>(out) = u32x4_a2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                       pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
        } else {
          const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gcol + e < p.N) out[e] = f32_to_bf16_bits(v[e]);
        }
      }
    }
  }
}

// The buffer range check works per requested dword, so when N % 4 != 0 the
// 16-byte load holding the last columns of B's last row returns its final
// N % 4 valid bytes as zeros (they share a dword with bytes past the
// window).  The tile holding column N-1 adds those products afterwards:
// columns c = N - N%4 .. N-1 sit in one 4-column group, held by the lanes
// with l/16 == (c - n0) % 16 / 4 of block j == (c - n0) % 64 / 16 of wave
// column (c - n0) / 64, as elements e = c % 4 of each of their rows.
template <int FM>
__device__ __forceinline__ void add_tail_products(f32x4 (&acc)[FM][kFN], const Fp8Args& p, int row0,
                                                  int n0, int wn, int lane, int hb) {
  const int c0 = p.N - (p.N & 3) - n0;  // first column of the group, within the tile
  if (wn != c0 / 64 || (lane >> 4) != (c0 % 16) / 4) return;
  const int jt = (c0 % 64) / 16;
  const int g = p.G - 1;
  const uint8_t* brow = p.B + static_cast<int64_t>(p.K - 1) * p.N + n0 + c0;
  float bv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) bv[e] = e < (p.N & 3) ? e4m3_value(brow[e]) : 0.0f;
  const float sb = hb < p.H ? p.sB[static_cast<int64_t>(g) * p.H + hb] : 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = row0 + (lane & 15) + 16 * i;
    if (row >= p.M) continue;
    const float a = e4m3_value(p.A[static_cast<int64_t>(row) * p.K + p.K - 1]) *
                    p.sA[static_cast<int64_t>(row) * p.G + g] * sb;
#pragma unroll
    for (int j = 0; j < kFN; ++j)
      if (j == jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(a, bv[e], acc[i][j][e]);
  }
}

// Work split of one launch: workgroups [0, whole) own whole tiles (logical
// tiles 0 .. whole-1).  Then either (halves > 0) the next 2 * halves
// workgroups own the 128-row halves of logical tiles whole .. whole +
// halves - 1 (two per tile, over all of K: the last round of tiles fills
// twice as many compute units, and every output element sees the same MFMAs
// and folds in the same order, so the result is bit-identical), or the next
// split_tiles * parts workgroups own part q of logical tile whole + t.
// part: parts * split_tiles partial tiles of kBM * kBN fp32; count:
// split_tiles counters, zero between calls.
struct SplitTail {
  int whole;
  int split_tiles;
  int parts;
  f32x4* part;
  uint32_t* count;
  int halves;
};

// BT: B given as [N, K] (K-contiguous rows, the nn.Linear weight layout);
// its tile is then loaded, stored and read exactly like A's, and its MFMA
// operands carry the same bytes as the [K, N] path's transposed reads.
// KFULL: K is a multiple of 128, so every slice inside K is whole and the
// loads need no per-lane column check (measured 1-2 % faster); slices past
// K read zeros through an out-of-range offset (A and a [N, K] B) or by
// lying past the window ([K, N] B).
// WHOLE (the launcher's choice when every offset of the call stays below
// 2^31): one window per operand and one for the tile's A scales cover all of
// K, built and made uniform once, and each slice's K offset rides in the
// per-lane offset, instead of three windows built per slice (1 % on the
// median, 3 % on the mean of the 4096 x 14336 x 4096 calls).  Otherwise the
// windows of slice g start at its K offset and end past K.
// One workgroup's share: the BM rows m0 .. of the 256 columns n0 .. (a
// whole tile or a half, Fp8Shape), over scale groups [g0, g1) -- part kpart
// of `parts` of logical tile `logical` when parts > 1.
template <int BM, bool BT, bool KFULL, bool WHOLE>
__device__ __forceinline__ void fp8_tile(const Fp8Args& p, const SplitTail& st, int logical, int kpart,
                                         int parts, int m0, int n0, uint8_t* smem, float (*s_sa)[kBM],
                                         int* s_last) {
  using T = Fp8Shape<BM>;
  constexpr int kFM = T::kFM;
  constexpr int kWTM = T::kWTM;
  constexpr int kAStage = T::kAStage;
  constexpr int kStage = T::kStage;
  constexpr int kSlots = T::kSlots;
  constexpr int kBar = T::kBar;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int g0 = static_cast<int>(static_cast<int64_t>(p.G) * kpart / parts);
  const int g1 = static_cast<int>(static_cast<int64_t>(p.G) * (kpart + 1) / parts);
  const int hb = (n0 + wn * kWTN) / 128;  // this wave's B-scale column

  // acc[i][j]: 16 x 16 block, transposed by the operand swap: element e of
  // lane l is row 16*i + l%16, column 16*j + 4*(l/16) + e of the wave tile.
  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{};

  // ---- global -> LDS.  Block b < 32 holds A rows 8b .. 8b+7, block
  // 32 + b holds B rows 4b .. 4b+3; slot 64b + lane holds chunk
  // (slot % chunks-per-row) ^ swizzle(row) of its row. ----
  const bool loads_a = wave < 4;
  const bool a_like = loads_a || BT;  // rows are K-contiguous, 8 per block
  const int blk0 = (wave & 3) * (loads_a ? T::kABlocks : kBBlocks);
  // A block blk (rows 8 blk .. +7): slot 64 blk + lane is row 8 blk + lane/8,
  // physical chunk lane % 8, logical chunk (lane % 8) ^ a_swz(row), and
  // a_swz(row) = (lane/8) ^ (blk & 1) takes two forms by the parity of blk.
  // B block blk (K rows 4 blk .. +3): row 4 blk + lane/16, physical chunk
  // lane % 16, and b_swz(row) likewise has two forms by the parity of blk
  // (bit 3 of it is (wave & 3) & 1 for every block of this wave).  The row
  // offset of the block is a wave-uniform addend, so a lane keeps only its
  // two in-block offsets.  With BT, B blocks hold 8 rows of [N, K] like A's.
  int lc[2];       // logical chunk for even / odd blocks
  uint32_t vo[2];  // in-block byte offset for even / odd blocks
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    if (a_like) {
      lc[par] = (lane & 7) ^ a_swz(8 * par + (lane >> 3));
      vo[par] = static_cast<uint32_t>((lane >> 3) * p.K + 16 * lc[par]);
    } else {
      lc[par] = (lane & 15) ^ (((4 * par + (lane >> 4)) & 7) | (((wave & 3) & 1) << 3));
      vo[par] = static_cast<uint32_t>((lane >> 4) * p.N + 16 * lc[par]) |
                (n0 + 16 * lc[par] < p.N ? 0u : kOutOfRange);
    }
  }
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  const uint32_t ssa_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(float, &s_sa[0][0])));
  // The wave's own matrix, slice by slice: the buffer window of slice g
  // starts at win0 + g * wstep and spans wsize0 - g * wstep bytes (A rows
  // m0 .. M-1 from column 128 g; B rows 128 g .. K-1 from column n0), so
  // bytes past M or K read as zeros.
  const uint8_t* win0 = loads_a ? p.A + static_cast<int64_t>(m0) * p.K
                                : (BT ? p.B + static_cast<int64_t>(n0) * p.K : p.B + n0);
  const int64_t wsize0 = loads_a ? static_cast<int64_t>(p.M - m0 - 1) * p.K + p.K
                                 : (BT ? static_cast<int64_t>(p.N - n0 - 1) * p.K + p.K
                                       : static_cast<int64_t>(p.K - 1) * p.N + (p.N - n0));
  const int64_t wstep = a_like ? int64_t{kBK} : int64_t{kBK} * p.N;
  const uint32_t blk_stride = a_like ? 8u * p.K : 4u * p.N;  // bytes per block of rows
  i32x4 w_all{}, sa_all{};
  if constexpr (WHOLE) {
    w_all = uniform_words(make_window_words(win0, wsize0));
    sa_all = uniform_words(make_window_words(p.sA + static_cast<int64_t>(m0) * p.G,
                                             static_cast<int64_t>(p.M - m0) * p.G * 4));
  }
  const uint32_t wstep32 = static_cast<uint32_t>(wstep);
  auto window = [&](int g) {
    if constexpr (WHOLE) return w_all;
    else if constexpr (KFULL) return make_window_words(win0 + g * wstep, g < p.G ? wsize0 - g * wstep : 0);
    else return make_window_words(win0 + g * wstep, wsize0 - g * wstep);
  };
  // Waves 0 .. BM/64 - 1 also fetch the scale column sA[m0 + 64*wave + lane, g].
  const uint32_t sa_off = static_cast<uint32_t>((64 * (wave & 3) + lane) * p.G * 4);
  const int64_t sa_size = (static_cast<int64_t>(p.M - m0 - 1) * p.G + 1) * 4;
  // A loads past K read zeros: kc is the chunk's first column for A waves
  // and a large negative number for B waves (no column check).
  int kc[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) kc[par] = a_like ? 16 * lc[par] : -(1 << 30);
  const uint32_t dst0 = smem_base + (loads_a ? 0u : static_cast<uint32_t>(kAStage)) +
                        static_cast<uint32_t>(blk0) * 1024u;
  const uint32_t off0 = static_cast<uint32_t>(blk0) * blk_stride;
  // This wave's i-th block of slice g.  Slices g >= G are allowed (they read
  // zeros: their windows are empty past K) so the schedule needs no branch.
  auto issue = [&](i32x4 w, int g, int i) {
    uint32_t off = vo[i & 1] + off0 + static_cast<uint32_t>(i) * blk_stride;
    if constexpr (WHOLE) off += static_cast<uint32_t>(g) * wstep32;  // keeps a column's out-of-range bit
    if constexpr (!KFULL) off |= g * kBK + kc[i & 1] < p.K ? 0u : kOutOfRange;
    else if (WHOLE && a_like) off |= g < p.G ? 0u : kOutOfRange;
    const uint32_t lds = dst0 + static_cast<uint32_t>((g & 1) * kStage + i * 1024);
    if constexpr (WHOLE) buf_load16_lds_u(w, lds, off);
    else buf_load16_lds(w, lds, off);
  };
  auto issue_scales = [&](int g) {
    if (wave < BM / 64) {
      const uint32_t lds = ssa_base + ((g & 1) * kBM + 64 * wave) * 4;
      if constexpr (WHOLE) {
        buf_load4_lds_u(sa_all, lds, (sa_off + 4u * static_cast<uint32_t>(g)) | (g < p.G ? 0u : kOutOfRange));
      } else {
        const i32x4 w = make_window_words(p.sA + static_cast<int64_t>(m0) * p.G + g, g < p.G ? sa_size : 0);
        buf_load4_lds(w, lds, sa_off);
      }
    }
  };
  // The tile holding column N-1 adds the products that the range check
  // drops from B's last row (add_tail_products).
  const bool tail_tile = !BT && (p.N & 3) != 0 && n0 + kBN >= p.N;

  // ---- LDS -> registers ----
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  // A operand of row block i: row wm*128 + 16i + l16, K bytes 32 lq .. +31
  // (chunks 2 lq and 2 lq + 1).  The swizzle depends only on l16.
  const int a_row = wm * kWTM + l16;
  const int a_off0 = a_row * kBK + (((2 * lq) ^ a_swz(l16)) * 16);
  const int a_off1 = a_row * kBK + (((2 * lq + 1) ^ a_swz(l16)) * 16);
  // B operand of column block j: column chunk cj = 4 wn + j; transposed read
  // s covers K rows 32 lq + 8 s + e for lane 16 lq + 2 e + h, columns 8 h .. +7.
  // BT: column block j is row block 4 wn + j of the [N, K] tile, read like
  // an A operand (b_off[0], b_off[1]: its two chunks in block 0).
  const int be = l16 >> 1, bh = l16 & 1;
  int b_off[kFN];
  if constexpr (BT) {
    const int b_row = wn * kWTN + l16;
    b_off[0] = kAStage + b_row * kBK + (((2 * lq) ^ a_swz(l16)) * 16);
    b_off[1] = kAStage + b_row * kBK + (((2 * lq + 1) ^ a_swz(l16)) * 16);
    b_off[2] = b_off[3] = 0;
  } else {
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int k = 32 * lq + be;
      b_off[j] = kAStage + k * kBN + (((4 * wn + j) ^ b_swz(k)) * 16) + 8 * bh;
    }
  }
  i32x8 fb[kFN];
  i32x8 fa[2];
  float srow[2];  // sA of the row block whose FMAs are pending / next (times sB at fold)
  f32x4 part[kFN];
  auto read_b = [&](int stage, int j) {
    if constexpr (BT) {
      const uint8_t* base = smem + stage * kStage + 16 * j * kBK;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(base + b_off[0]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(base + b_off[1]);
      fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
      const uint8_t* base = smem + stage * kStage + b_off[j];
      i32x2 q[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        q[s] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(TGEMM_LDS(i32x2, base + s * 8 * kBN));
      fb[j] = i32x8{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
    }
  };
  auto read_a = [&](int stage, int i) {
    const uint8_t* base = smem + stage * kStage + 16 * i * kBK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + a_off0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + a_off1);
    fa[i & 1] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto read_scale = [&](int stage, int i) { srow[i & 1] = s_sa[stage][a_row + 16 * i]; };
  // FMAs of block (i, j) from the partial sum of its last MFMA.
  auto fold = [&](int i, int j, float scale) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(part[j][e], scale, acc[i][j][e]);
  };

  const int G = p.G;
  if (g1 > g0) {
    // B scales of this wave's column block, 64 groups per register: lane l
    // holds sB[g0 + l, hb] and each group's value is taken with readlane.
    auto sb_fetch = [&](int g0) {
      const int gl = g0 + lane;
      return (gl < G && hb < p.H) ? p.sB[static_cast<int64_t>(gl) * p.H + hb] : 0.0f;
    };
    auto sb_of = [&](float lanes, int g) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lanes), g & 63));
    };
    // The first slice folds a zero "previous row".
#pragma unroll
    for (int j = 0; j < kFN; ++j) part[j] = f32x4{};
    srow[1] = 0.0f;
    float sb_lanes = sb_fetch(g0 & ~63);
    float sb_cur = sb_of(sb_lanes, g0);
    // Prologue: slice g0, then the first kEarly blocks of slice g0+1.
    {
      const i32x4 w = window(g0);
#pragma unroll
      for (int i = 0; i < kBBlocks; ++i)
        if (i < T::kABlocks || !loads_a) issue(w, g0, i);
      issue_scales(g0);
    }
    if (g1 - g0 > 1) {
      const i32x4 w = window(g0 + 1);
#pragma unroll
      for (int i = 0; i < kEarly; ++i) issue(w, g0 + 1, i);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kEarly) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();
    // Same order as the reads of the next slice in the last row of the loop.
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      read_b(g0 & 1, j);
      if (j == 0) read_a(g0 & 1, 0);
      if (j == 1) read_scale(g0 & 1, 0);
    }

    float sb_prev = 0.0f;  // sB of the slice whose last row is pending
    float scale = 0.0f;    // sA * sB of the row being folded
    for (int g = g0; g < g1; ++g) {
      const int stage = g & 1;
      if (((g + 1) & 63) == 0) {
        // Next 64 B scales; wait here (rarely) rather than at their use,
        // where the wait would also cover the slices in flight.
        sb_lanes = sb_fetch(g + 1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
      const i32x4 w1 = window(g + 1);
      const i32x4 w2 = window(g + 2);
      float sb_next = 0.0f;
      static_for<kSlots>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int i = s / kFN, j = s % kFN;
        if constexpr (s == kBar) {
          // Slice g+1 has landed and every wave is done reading slice g's
          // stage (all its operands for this last row are in registers).
          TGEMM_SCHED_FENCE();
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          lds_barrier();
          sb_next = sb_of(sb_lanes, g + 1);
        }
        TGEMM_SCHED_FENCE();
        // FMAs of the previous row (row kFM-1 of the previous slice at i == 0).
        if constexpr (j == 0) scale = srow[(i + 1) & 1] * (i == 0 ? sb_prev : sb_cur);
        fold(i == 0 ? kFM - 1 : i - 1, j, scale);
        part[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[j], fa[i & 1], f32x4{}, kFmtE4M3, kFmtE4M3, 0, kScaleOne, 0, kScaleOne);
        TGEMM_SCHED_FENCE();
        // Operand reads.
        if constexpr (i + 1 < kFM) {
          if constexpr (j == 0) read_a(stage, i + 1);
          if constexpr (j == 1) read_scale(stage, i + 1);
        } else {
          read_b(stage ^ 1, j);  // fb[j] of slice g+1 replaces the one just used
          if constexpr (j == 0) read_a(stage ^ 1, 0);
          if constexpr (j == 1) read_scale(stage ^ 1, 0);
        }
        // Global -> LDS: blocks kEarly.. of slice g+1 in the first slots,
        // blocks 0 .. kEarly-1 of slice g+2 right after the barrier.
        if constexpr (s < kBBlocks - kEarly) {
          if (kEarly + s < T::kABlocks || !loads_a) issue(w1, g + 1, kEarly + s);
        }
        if constexpr (s == kBBlocks - kEarly) issue_scales(g + 1);
        if constexpr (s >= kBar && s < kBar + kEarly) issue(w2, g + 2, s - kBar);
      });
      TGEMM_SCHED_FENCE();
      sb_prev = sb_cur;
      sb_cur = sb_next;
    }
    // FMAs of the last row of the last slice.
    scale = srow[1] * sb_prev;
#pragma unroll
    for (int j = 0; j < kFN; ++j) fold(kFM - 1, j, scale);
    if (tail_tile && g1 == G) add_tail_products(acc, p, m0 + wm * kWTM, n0, wn, lane, hb);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (BM == kBM && parts > 1) {
    // Publish this part's fp32 partial tile (lane-contiguous 16-byte
    // stores), then count the parts that are done; only the last one goes on.
    const int t = logical - st.whole;
    f32x4* const part0 = st.part + static_cast<int64_t>(t) * parts * (kFM * kFN * kThreads);
    f32x4* const mine = part0 + static_cast<int64_t>(kpart) * (kFM * kFN * kThreads);
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) mine[(i * kFN + j) * kThreads + tid] = acc[i][j];
    // Every wave's stores have reached L2 before the barrier; thread 0's
    // release then writes them back for the other dies, once per workgroup
    // (a device-scope fence in every wave would write back and invalidate
    // the die's L2 eight times over).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t done =
          __hip_atomic_fetch_add(st.count + t, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int last = done + 1 == static_cast<uint32_t>(parts);
      // The last part resets the counter for the next call.
      if (last) __hip_atomic_store(st.count + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = last;
    }
    __syncthreads();  // thread 0's acquire (cache invalidation) precedes every wave's reads
    if (!*s_last) return;
    // Sum in part order, ((P0 + P1) + P2) + ..., all read back from the
    // scratch (this part's own as well), so the bits do not depend on which
    // part came last.
    // One part at a time, its 32 loads issued together.
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = part0[(i * kFN + j) * kThreads + tid];
    for (int q = 1; q < parts; ++q) {
      const f32x4* src = part0 + static_cast<int64_t>(q) * (kFM * kFN * kThreads) + tid;
      f32x4 v[kFM][kFN];
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) v[i][j] = src[(i * kFN + j) * kThreads];
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] += v[i][j];
    }
  }
  lds_barrier();  // every wave is done with the operand stages

  // ---- epilogue ----
  store_wave(acc, reinterpret_cast<float*>(smem) + wave * 16 * kEpiPitch, lane, m0 + wm * kWTM,
             n0 + wn * kWTN, p);
}

template <bool BT, bool KFULL, bool WHOLE>
__global__ __launch_bounds__(kThreads, 1) void tgemm_fp8_bs_256x256x128(Fp8Args p, int tiles_m,
                                                                     int tiles_n, SplitTail st) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * Fp8Whole::kStage];
  __shared__ __attribute__((aligned(256))) float s_sa[2][kBM];
  __shared__ int s_last;

  // Tile, tile half and K range of this workgroup (SplitTail).
  const int bid = blockIdx.x;
  int logical, kpart = 0, parts = 1, half = -1;
  if (bid < st.whole) {
    logical = xcd_remap(bid, st.whole);
  } else if (st.halves > 0) {
    const int r = xcd_remap(bid - st.whole, 2 * st.halves);
    logical = st.whole + r / 2;
    half = r & 1;
  } else {
    const int r = xcd_remap(bid - st.whole, st.split_tiles * st.parts);
    logical = st.whole + r / st.parts;
    kpart = r % st.parts;
    parts = st.parts;
  }
  int tm, tn;
  tile_coords(logical, tiles_m, tiles_n, kGroupM, tm, tn);
  const int n0 = tn * kBN;
  if (half < 0) {
    fp8_tile<kBM, BT, KFULL, WHOLE>(p, st, logical, kpart, parts, tm * kBM, n0, smem, s_sa, &s_last);
  } else {
    // A tile row of at most 128 rows (the last, when M % 256 <= 128) has
    // nothing in its second half: that workgroup ends at once.
    const int m0 = tm * kBM + half * (kBM / 2);
    if (m0 < p.M) fp8_tile<kBM / 2, BT, KFULL, WHOLE>(p, st, logical, 0, 1, m0, n0, smem, s_sa, &s_last);
  }
}


}  // namespace

bool fp8_direct_ok(int64_t M, int64_t N, int64_t K) {
  (void)M;
  // N >= 4: below that one 4-byte word of B spans more than two rows, and
  // the last-row patch would not cover every zeroed byte.
  return K % 16 == 0 && N >= 4 && K * kBM < (int64_t{1} << 31) && N * kBK < (int64_t{1} << 31) &&
         static_cast<int64_t>(kBM) * ((K + 127) / 128) * 4 < (int64_t{1} << 31);
}

bool fp8_nt_ok(int64_t M, int64_t N, int64_t K) {
  (void)M;
  // Per-lane offsets: a tile's 256 rows of A and of Bt.
  return K % 16 == 0 && K * kBM < (int64_t{1} << 31) && K * kBN < (int64_t{1} << 31) &&
         static_cast<int64_t>(kBM) * ((K + 127) / 128) * 4 < (int64_t{1} << 31);
}

const char* fp8_kernel_name(int64_t M, int64_t N, int64_t K) {
  return fp8_direct_ok(M, N, K) ? "tgemm_fp8_bs_256x256x128" : "tgemm_fp8_bs_general_256x128x128";
}

Fp8Split fp8_split_plan(int64_t M, int64_t N, int64_t K, int cus, int forced_parts) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int64_t G = (K + 127) / 128;
  Fp8Split plan{static_cast<int>(tiles), 0, 1};
  if (cus <= 0 || tiles == 0 || forced_parts == 1 || !fp8_direct_ok(M, N, K)) return plan;
  const int64_t left = tiles - (tiles - 1) / cus * cus;  // tiles of the last round
  int64_t parts;
  if (forced_parts >= 2) {
    parts = forced_parts < G ? forced_parts : G;  // at least one scale group per part
  } else {
    // Measured on MI355X: splitting pays only when at most a quarter of the
    // compute units would be busy (1 .. 32 tiles ran 1.2 - 3.5x faster; 128
    // tiles, or the 128-tile last round of a 4096 x 14336 grid, ran 2 - 18 %
    // slower, as a partly idle chip runs each tile faster), with at least
    // eight scale groups per part (fewer leave the partial-tile traffic and
    // the fixup exposed).
    if (tiles > left || 4 * left > cus) return plan;
    parts = cus / left;
    if (parts > kFp8MaxParts) parts = kFp8MaxParts;
    if (parts > G / 8) parts = G / 8;
  }
  if (parts < 2 || left > kFp8MaxSplitTiles) return plan;
  plan.whole = static_cast<int>(tiles - left);
  plan.split_tiles = static_cast<int>(left);
  plan.parts = static_cast<int>(parts);
  return plan;
}

size_t fp8_split_part_bytes(const Fp8Split& plan) {
  return static_cast<size_t>(plan.split_tiles) * plan.parts * kBM * kBN * sizeof(float);
}

// Whole-K windows fit when every per-lane offset stays below 2^31: a
// tile's 256 rows of A (or of a [N, K] B) plus the slice offsets up to two
// slices past K, or for a [K, N] B all of its rows up to three slices past
// K.
static bool fp8_whole_windows_ok(const Fp8Args& a) {
  const int64_t lim = int64_t{1} << 31;
  const int64_t rows = (int64_t{kBM} + 1) * a.K + 4 * kBK;  // A, and B given as [N, K]
  if (rows >= lim) return false;
  return a.bt || (static_cast<int64_t>(a.K) + 3 * kBK) * a.N + 4 * kBK < lim;
}

template <bool BT, bool KFULL>
static hipError_t launch_fp8_w(const Fp8Args& a, bool whole, dim3 grid, int tiles_m, int tiles_n,
                               const SplitTail& st, hipStream_t s) {
  if (whole)
    hipLaunchKernelGGL((tgemm_fp8_bs_256x256x128<BT, KFULL, true>), grid, dim3(kThreads), 0, s, a, tiles_m, tiles_n, st);
  else
    hipLaunchKernelGGL((tgemm_fp8_bs_256x256x128<BT, KFULL, false>), grid, dim3(kThreads), 0, s, a, tiles_m, tiles_n, st);
  return hipGetLastError();
}

int fp8_tail_halves(int64_t tiles, int cus) {
  if (cus <= 0 || tiles <= 0) return 0;
  const int64_t left = tiles - (tiles - 1) / cus * cus;  // tiles of the last round
  return 2 * left <= cus ? static_cast<int>(left) : 0;
}

hipError_t launch_fp8_blockscaled(const Fp8Args& a, const Fp8Split& plan, void* part, uint32_t* count,
                                  bool halves, hipStream_t s) {
  if (a.bt && !fp8_nt_ok(a.M, a.N, a.K)) return hipErrorInvalidValue;
  if (!a.bt && !fp8_direct_ok(a.M, a.N, a.K)) return launch_fp8_general(a, s);
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles_n = (a.N + kBN - 1) / kBN;
  const int tiles = tiles_m * tiles_n;
  SplitTail st{tiles, 0, 1, nullptr, nullptr, 0};
  if (plan.parts > 1 && part != nullptr && count != nullptr && plan.whole + plan.split_tiles == tiles) {
    st.whole = plan.whole;
    st.split_tiles = plan.split_tiles;
    st.parts = plan.parts;
    st.part = static_cast<f32x4*>(part);
    st.count = count;
  } else if (halves) {
    // A last round of whole tiles that would leave at least half of the
    // compute units idle runs as twice as many 128-row halves instead (the
    // 4096 x 14336 grid's 3.5 rounds become 3 + one full round of halves:
    // 4.6 % faster on MI355X; grids of 64 or 128 tiles 22-26 %).
    st.halves = fp8_tail_halves(tiles, device_cus());
    st.whole = tiles - st.halves;
  }
  const dim3 grid(st.whole + (st.halves > 0 ? 2 * st.halves : st.split_tiles * st.parts));
  const bool kfull = a.K % kBK == 0;
  const bool whole = fp8_whole_windows_ok(a);
  if (a.bt) {
    if (kfull) return launch_fp8_w<true, true>(a, whole, grid, tiles_m, tiles_n, st, s);
    return launch_fp8_w<true, false>(a, whole, grid, tiles_m, tiles_n, st, s);
  }
  if (kfull) return launch_fp8_w<false, true>(a, whole, grid, tiles_m, tiles_n, st, s);
  return launch_fp8_w<false, false>(a, whole, grid, tiles_m, tiles_n, st, s);
}

}  // namespace tgemm
