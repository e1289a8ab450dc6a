// Small-M GEMMs with integer weights and per-group fp32 scales (weight-only
// quantisation) for gfx950, written as bandwidth-bound kernels.
//
//   C[i, n] = epilogue( sum_k X[i, k] * (q[k, n] * S[k / 128, n]) + bias[n] )
//
// The GEMM compute-cost page (section 7.2, the LM head) names keeping the
// large output projection in a low-precision integer format as the first
// remedy for its memory-bound cost: the weight W[K, N] is streamed once per
// call, so halving its bytes halves the time (section 4.3 of the same page
// lists int8 and int4 as the usual formats).  W is stored as integer codes
// q with one fp32 scale per (128-row group along K, column), the
// round-to-nearest per-group scheme of the DeepGEMM page's section 2.4
// applied to integers; activations X stay bf16.  Two code widths:
//   * int8: Q [K, N] bytes, one signed code per byte;
//   * int4: Q [K/2, N] bytes, two signed 4-bit codes per byte along K (byte
//     (r, n) holds q[2r, n] in its low nibble and q[2r+1, n] in its high
//     nibble, two's complement, codes -8 .. 7).
//
// Layout of the work (the bf16 thin-M kernel's, with byte rows):
//   * a workgroup owns 512 consecutive columns: a byte row of its stripe is
//     512 contiguous bytes; the stripe is walked in slices of 32 byte rows
//     (32 K rows of int8, 64 of int4), each with the matching 16-row blocks
//     of X and the 512 scales of the slice's group, one load instruction
//     per two byte rows.  In the full-width kernels, int8 slices for up to
//     48 rows of X and int4 slices for up to 32 go through registers (four
//     slices in flight per wave, codes with the non-temporal hint) into two
//     LDS stages; more rows and the split-K kernel go global -> LDS with
//     direct buffer loads, six LDS stages deep;
//   * eight waves (two per SIMD) each own 64 columns over the whole of K.
//     A wave's MFMA operand for 16 columns comes from one ds_read_b64_tr_b8
//     (lane i receives column i of 8 byte rows: the 8 K values one
//     16 x 16 x 32 MFMA takes per lane for int8, those of two MFMAs for
//     int4); every code becomes a bf16 exactly (a sign-extending byte to fp32
//     conversion, then the upper half; an int4 code goes through the 4-bit
//     signed conversion, which gives q / 16, and the 16 goes into the group
//     scale).  The conversions of one 16-column block are placed by hand
//     between the MFMAs of the previous one, so each wave keeps the matrix
//     unit and the vector unit busy together (the two waves of a SIMD leave
//     each slice's barrier in step, so they rarely cover each other);
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
constexpr int kRows = 32;       // byte rows of Q per slice
constexpr int kGroupK = 128;    // K rows per scale group
constexpr int kNS = 6;          // LDS stages
constexpr int kWRow = kBN;      // bytes per Q row of the stripe
constexpr int kWStage = kRows * kWRow;   // 16 KiB
constexpr int kSStage = kBN * 4;         // the slice group's 512 fp32 scales
constexpr int kLoadsPerSlice = 2 + 1 + 1;  // per wave: 4 Q rows, one KiB of X, 64 scales

// Per code width: K rows per slice (kBK), bytes of one 16-row X block of a
// slice, the X part of a stage (four blocks) and the stage size.
template <int BITS>
struct WqShape {
  static_assert(BITS == 8 || BITS == 4, "int8 or int4 codes");
  static constexpr int kBK = kRows * 8 / BITS;
  static constexpr int kXBlock = 16 * kBK * 2;
  static constexpr int kXStage = 4 * kXBlock;
  static constexpr int kStage = kWStage + kXStage + kSStage;
  static constexpr int kSlicesPerGroup = kGroupK / kBK;
  // Slices between barriers: int4 slices carry twice the conversion work
  // of int8 ones, and two per barrier let a wave's conversions of one run
  // into the other's (measured 5-10 % faster for int4, 0-5 % slower for
  // int8).
  static constexpr int kPerBar = BITS == 4 ? 2 : 1;
  static_assert(kNS * kStage <= 160 * 1024, "LDS capacity");
};

// Load pipeline: the full-width kernels stream int8 slices for up to 48 rows
// of X and int4 slices for up to 32 through registers into two LDS stages.
// More rows (whose four register slices would not fit beside the group
// partials and accumulators in a wave's 256 registers) and the split-K
// kernel (whose short chunks gain more from depth) load straight into LDS,
// kNS stages deep.
template <int BITS, int MB, bool SPLIT = false>
struct WqStages {
  static constexpr bool kRegisters = !SPLIT && MB <= (BITS == 8 ? 3 : 2);
  static constexpr int kCount = kRegisters ? 2 : kNS;
};

#define TGEMM_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// XOR on the 16-byte chunk index of byte row k of a Q slice, so that the 16
// byte rows one transposed read covers per 32 lanes land in 16 different
// 16-byte bank slots of a 256-byte bank row.  int8: rows 8g + e (g < 2,
// e < 8).  int4: rows 4g + e and 16 + 4g + e (g < 2, e < 4) -- the K values
// 8g .. 8g+7 of the slice's two 32-wide MFMA steps.
template <int BITS>
__device__ __forceinline__ int q_swz(int k) {
  if constexpr (BITS == 8) return k & 15;
  else return (k & 7) | (((k >> 4) & 1) << 3);
}
// XOR on the chunk index of row r of an X block: 4 chunks per row (int8
// slices, 64-byte rows) or 8 (int4 slices, 128-byte rows); the 16 rows one
// operand read covers land in distinct 16-byte slots.
template <int BITS>
__device__ __forceinline__ int x_swz(int r) {
  if constexpr (BITS == 8) return (r >> 2) & 3;
  else return (r >> 1) & 7;
}

// 4-byte buffer load written straight into LDS (lane l -> lds_base + 4 l).
__device__ __forceinline__ void buf_load4_lds(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_words(window))
               : "memory", "m0");
}

// The 4-byte load for a descriptor already made uniform (as
// buf_load16_lds_u): a readfirstlane per load made the compiler keep the
// loop-invariant descriptors in vector registers and copy them back for
// every load (nine vector instructions per slice here, about 3 % of the int8
// head's time at 64 rows).
__device__ __forceinline__ void buf_load4_lds_u(i32x4 window, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(window)
               : "memory", "m0");
}

// int8 codes stream through registers (see wq_accumulate): one slice of
// one wave in flight is its two 16-byte Q loads, its X load and its scale.
constexpr int kRegSlices = 4;     // slices in flight per wave
constexpr uint32_t kCacheNT = 2;   // buffer-load cache policy: non-temporal
struct WqRegs {
  u32x4 q[2];
  u32x4 x;
  uint32_t s;
};

// Buffer descriptor over [base, base + bytes), bytes clamped to [0, 2^31 - 1]
// with 32-bit compares so the descriptor stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wq_window(const void* base, int64_t bytes) {
  const uint64_t u = static_cast<uint64_t>(bytes);
  const int32_t hi = static_cast<int32_t>(u >> 32);
  const uint32_t lo = static_cast<uint32_t>(u);
  const int32_t n = hi < 0 ? 0 : ((hi > 0 || lo > 0x7fffffffu) ? 0x7fffffff : static_cast<int32_t>(lo));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           static_cast<int>(kBufferFlags));
}

// Word o of eight int8 codes (two dwords, K order) as bf16, exactly: codes
// 2o and 2o + 1, each through a sign-extending byte to fp32 conversion, then
// the upper halves of the two fp32 words in one permute (1.5 vector
// instructions per code).
template <int O>
__device__ __forceinline__ uint32_t codes_pair_bf16(i32x2 codes) {
  const uint32_t w = static_cast<uint32_t>(codes[O >> 1]);
  const float a = static_cast<float>(static_cast<int8_t>(w >> (8 * ((2 * O) & 3))));
  const float b = static_cast<float>(static_cast<int8_t>(w >> (8 * ((2 * O + 1) & 3))));
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// q / 16 for the 4-bit two's-complement code in bits 0-3 of byte E of v,
// exactly: v_cvt_off_f32_i4 converts bits 0-3 of its operand that way, and
// the SDWA byte select picks the byte in the same instruction (the compiler
// would shift first; all 16 codes in all four bytes, low and shifted-down
// high nibbles, checked on the GPU against q / 16).
template <int E>
__device__ __forceinline__ float nibble_q16(uint32_t v) {
  float r;
  if constexpr (E == 0)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(v));
  if constexpr (E == 1)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(v));
  if constexpr (E == 2)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(v));
  if constexpr (E == 3)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(v));
  return r;
}

// Four bytes of int4 codes (byte e = K values 2e (low nibble), 2e + 1 (high
// nibble)) are 8 bf16 holding q / 16, exactly: one conversion per code (the
// high nibbles after one shift of the word, hi = codes >> 4), then the upper
// halves of two fp32 words per permute -- 13 vector instructions per 8 codes
// (moving each nibble to the top of its byte and converting the
// sign-extended byte, 16 q, took 15; 2-4 % slower at M = 1 ... 32).  This
// gives words 2H and 2H + 1 of the four.
template <int H>
__device__ __forceinline__ u32x2 nibble_words(uint32_t codes, uint32_t hi) {
  const float f0 = nibble_q16<2 * H>(codes), f1 = nibble_q16<2 * H>(hi);
  const float f2 = nibble_q16<2 * H + 1>(codes), f3 = nibble_q16<2 * H + 1>(hi);
  return u32x2{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u)};
}

// Streams the workgroup's 512-column stripe of Q once and leaves the scaled
// products in acc[mb][j] (16 x 16 blocks, transposed by the operand swap:
// element e of lane l is row 16*mb + l%16, column 16*j + 4*(l/16) + e of the
// wave's 64).  Slices [tb, te) of K (te < 0: through the last) are summed;
// a range starts and ends on a scale-group boundary (or at K), and its end
// acts as K, so nothing past it is loaded.  Ends with no load still writing
// LDS; the caller synchronises the workgroup before reusing smem.
template <int BITS, int MB, bool WHOLE, bool SPLIT = false>
__device__ __forceinline__ void wq_accumulate(const W8Args& p, uint8_t* smem, f32x4 (&acc)[MB][kFN], int tb = 0,
                                              int te = -1) {
  using Sh = WqShape<BITS>;
  constexpr int kBK = Sh::kBK;
  constexpr int kStage = Sh::kStage;
  constexpr int kXStage = Sh::kXStage;
  constexpr int NS = WqStages<BITS, MB, SPLIT>::kCount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kBN;

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[mb][j] = f32x4{};

  // ---- global -> LDS.  Q: load i of wave w covers slice byte rows 4w + 2i
  // (lanes 0-31) and 4w + 2i + 1 (lanes 32-63), lane -> physical chunk
  // lane % 32, logical chunk (lane % 32) ^ q_swz(row).  X, int8 (64-byte
  // rows): block w % 4 (rows 16(w%4) .. +15), lane -> row l/4, physical
  // chunk l%4 (waves 4-7 write the same bytes as waves 0-3, which keeps
  // every wave's load count equal).  X, int4 (128-byte rows): block w / 2,
  // rows 8(w%2) + l/8, physical chunk l%8.  Scales: wave w fetches columns
  // 64w .. 64w+63 of the group. ----
  const int64_t ldx2 = p.ldx * 2;
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TGEMM_LDS(uint8_t, smem)));
  // In-slice offset of this lane's Q chunk, with the out-of-range mark for
  // columns past N.  With a whole-stripe window the slice's row offset is
  // added to it: lanes of in-range columns stay below the window's end (under
  // 2^31); a marked lane stays at or above 2^31 unless the stripe ends within
  // 512 bytes of 2^31, where it may wrap into the window and fill LDS columns
  // past N, which no output reads.  Slices past the range land in stages
  // that are never read.
  uint32_t w_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = 4 * wave + 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ q_swz<BITS>(k);
    w_off[i] = static_cast<uint32_t>(k * p.ldq + 16 * c) | (n0 + 16 * c < p.N ? 0u : kOutOfRange);
  }
  // Row (within the four blocks) and logical chunk this lane loads of X.
  const int xr = BITS == 8 ? 16 * (wave & 3) + (lane >> 2) : 8 * wave + (lane >> 3);
  const int xc = BITS == 8 ? (lane & 3) ^ x_swz<BITS>(xr & 15) : (lane & 7) ^ x_swz<BITS>(xr & 15);
  const uint32_t x_off = static_cast<uint32_t>(xr * ldx2 + 16 * xc);
  const uint32_t x_dst = kWStage + (BITS == 8 ? (wave & 3) : wave) * 1024;
  const int KT = (p.K + kBK - 1) / kBK;
  if (te < 0) te = KT;
  const int kend = p.K < te * kBK ? p.K : te * kBK;  // this range's end of K
  const int G = (kend + kGroupK - 1) / kGroupK;       // groups up to it
  const int64_t q_rows = BITS == 8 ? kend : kend / 2;  // byte rows of Q up to it
  // Buffer windows.  WHOLE (the launcher's choice: the stripe's bytes of Q,
  // rows 0 .. K-1 from column 0, span less than 2^31): one window per
  // operand covers the whole range and each slice's row offset rides in the
  // per-lane offset; rows past the range, X rows past M and scale rows past
  // the range fall outside their window and read zeros.  That saves
  // rebuilding three descriptors per slice (about 60 scalar instructions;
  // 5-8 % faster on the 4096 x 128256 heads).  Otherwise each slice builds
  // its own windows.
  const int64_t q_span = (q_rows - 1) * p.ldq + (p.N - n0);
  // Made uniform here, once: the loads below take them as scalar operands.
  const i32x4 wq_all = uniform_words(make_window_words(p.Q + n0, q_span));
  const i32x4 wx_all = uniform_words(make_window_words(p.X, (static_cast<int64_t>(p.M - 1) * p.ldx + kend) * 2));
  const i32x4 ws_all =
      uniform_words(make_window_words(p.S + n0, (static_cast<int64_t>(G - 1) * p.N + (p.N - n0)) * 4));
  const uint32_t q_step = static_cast<uint32_t>(kRows * p.ldq);  // Q bytes per slice
  const uint32_t s_step = static_cast<uint32_t>(p.N * 4);        // scale bytes per group
  const uint32_t s_lane = static_cast<uint32_t>((64 * wave + lane) * 4);
  // Slice t into LDS stage st.
  auto issue_slice = [&](int t, int st) {
    const uint32_t stage = smem_base + static_cast<uint32_t>(st * kStage);
    const int k0 = t * kBK;
    const int g = k0 / kGroupK;
    const uint32_t x_tail = k0 + 8 * xc < kend ? 0u : kOutOfRange;
    if constexpr (WHOLE) {
      const uint32_t qo = static_cast<uint32_t>(t) * q_step;
#pragma unroll
      for (int i = 0; i < 2; ++i) buf_load16_lds_u(wq_all, stage + (4 * wave + 2 * i) * kWRow, w_off[i] + qo);
      buf_load16_lds_u(wx_all, stage + x_dst, (x_off + 2 * k0) | x_tail);
      buf_load4_lds_u(ws_all, stage + kWStage + kXStage + 64 * wave * 4, s_lane + static_cast<uint32_t>(g) * s_step);
    } else {
      const int64_t r0 = static_cast<int64_t>(t) * kRows;
      const i32x4 ww = make_window_words(p.Q + r0 * p.ldq + n0, (q_rows - r0 - 1) * p.ldq + (p.N - n0));
#pragma unroll
      for (int i = 0; i < 2; ++i) buf_load16_lds(ww, stage + (4 * wave + 2 * i) * kWRow, w_off[i]);
      const i32x4 wx = make_window_words(p.X + k0, (static_cast<int64_t>(p.M - 1) * p.ldx + (kend - k0)) * 2);
      buf_load16_lds(wx, stage + x_dst, x_off | x_tail);
      const i32x4 ws = make_window_words(p.S + static_cast<int64_t>(g) * p.N + n0,
                                         g < G ? static_cast<int64_t>(p.N - n0) * 4 : 0);
      buf_load4_lds(ws, stage + kWStage + kXStage + 64 * wave * 4, s_lane);
    }
  };
  // The same slice through registers: Q with the non-temporal hint (read
  // once by the whole grid), X and the scales cacheable; each lane's bytes
  // land in LDS where the direct loads above put them.
  const __amdgpu_buffer_rsrc_t rq_all = wq_window(p.Q + n0, q_span);
  const __amdgpu_buffer_rsrc_t rx_all = wq_window(p.X, (static_cast<int64_t>(p.M - 1) * p.ldx + kend) * 2);
  const __amdgpu_buffer_rsrc_t rs_all =
      wq_window(p.S + n0, (static_cast<int64_t>(G - 1) * p.N + (p.N - n0)) * 4);
  auto load_regs = [&](int t, WqRegs& r) {
    const int k0 = t * kBK;
    const int g = k0 / kGroupK;
    const uint32_t x_tail = k0 + 8 * xc < kend ? 0u : kOutOfRange;
    if constexpr (WHOLE) {
      const uint32_t qo = static_cast<uint32_t>(t) * q_step;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        r.q[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq_all, w_off[i] + qo, 0, kCacheNT));
      r.x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx_all, (x_off + 2 * k0) | x_tail, 0, 0));
      r.s = __builtin_amdgcn_raw_buffer_load_b32(rs_all, s_lane + static_cast<uint32_t>(g) * s_step, 0, 0);
    } else {
      const int64_t r0 = static_cast<int64_t>(t) * kRows;
      const __amdgpu_buffer_rsrc_t ww = wq_window(p.Q + r0 * p.ldq + n0, (q_rows - r0 - 1) * p.ldq + (p.N - n0));
#pragma unroll
      for (int i = 0; i < 2; ++i)
        r.q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ww, w_off[i], 0, kCacheNT));
      const __amdgpu_buffer_rsrc_t wx =
          wq_window(p.X + k0, (static_cast<int64_t>(p.M - 1) * p.ldx + (kend - k0)) * 2);
      r.x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wx, x_off | x_tail, 0, 0));
      const __amdgpu_buffer_rsrc_t ws = wq_window(p.S + static_cast<int64_t>(g) * p.N + n0,
                                                  g < G ? static_cast<int64_t>(p.N - n0) * 4 : 0);
      r.s = __builtin_amdgcn_raw_buffer_load_b32(ws, s_lane, 0, 0);
    }
  };
  auto store_regs = [&](int t, const WqRegs& r) {
    uint8_t* st = smem + (t % NS) * kStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(st + (4 * wave + 2 * i) * kWRow + 16 * lane) = r.q[i];
    *reinterpret_cast<u32x4*>(st + x_dst + 16 * lane) = r.x;
    *reinterpret_cast<uint32_t*>(st + kWStage + kXStage + 64 * wave * 4 + 4 * lane) = r.s;
  };

  // ---- LDS -> registers ----
  // Q operand of block j (columns 16 j .. +15 of the wave): within each
  // 16-lane group g, lane 2e + h supplies bytes 8h .. 8h+7 of the block in
  // byte row k(g, e) and receives column (lane % 16) of those 8 rows:
  // int8 rows 8g + e (K values 8g .. 8g+7); int4 rows 4g + e for e < 4 and
  // 16 + 4g + e - 4 for e >= 4 (K values 8g .. 8g+7 of MFMA steps 0 and 1).
  const int bg = lane >> 4, be = (lane >> 1) & 7, bh = lane & 1;
  int b_off[kFN];
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int k = BITS == 8 ? 8 * bg + be : 4 * bg + (be & 3) + 16 * (be >> 2);
    b_off[j] = k * kWRow + (((4 * wave + j) ^ q_swz<BITS>(k)) * 16) + 8 * bh;
  }
  // Scales of this lane's accumulator columns 16 j + 4 (lane / 16) .. +3.
  const int s_rd = kWStage + kXStage + (kWTN * wave + 4 * (lane >> 4)) * 4;
  // X operand of block mb and MFMA step u: row l%16, K 32u + 8*(l/16) .. +7
  // of the slice.
  const int xrow = lane & 15;
  int x_rd[kBK / 32];
#pragma unroll
  for (int u = 0; u < kBK / 32; ++u)
    x_rd[u] = kWStage + xrow * (kBK * 2) + (((4 * u + (lane >> 4)) ^ x_swz<BITS>(xrow)) * 16);
  // int4 operands carry q / 16.
  constexpr float kCodeScale = BITS == 8 ? 1.0f : 16.0f;

  if (te > tb) {
    f32x4 part[MB][kFN];  // sum over the current 128-row group of x * q
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < kFN; ++j) part[mb][j] = f32x4{};
    // One slice's operand reads, conversions and MFMAs, and the group fold
    // when it ends a 128-row group or the range.  A slice at or past te (the
    // partner of an odd last slice of a pair) reads zeros and adds nothing.
    // kZeroStart (int8 slices loaded straight into LDS): a group's first
    // slice starts its MFMAs from a zero accumulator instead of the fold
    // clearing the partial sums (one move per accumulator and group: 4-5 %
    // of the int8 head's time at 64 rows).  int4 and the register-staged
    // pipelines keep the clearing fold: there the zero start measured
    // slower (int4 3-5 %, also with the group's first slice known at
    // compile time) or no faster.
    constexpr bool kZeroStart = !WqStages<BITS, MB, SPLIT>::kRegisters && BITS == 8;
    // pos: the slice's place in its group when known at compile time (the
    // group-unrolled loop below), -1 when it follows from t.
    auto process = [&](int t, int st, auto pos) {
      constexpr int kPos = decltype(pos)::value;
      static_assert(!kZeroStart || kPos >= 0, "the zero start needs the slice's place in its group");
      const uint8_t* base = smem + st * kStage;
      constexpr int kSteps = kBK / 32;  // 16 x 16 x 32 MFMA steps per slice
      // Operands: the codes of the wave's kFN column blocks (one transposed
      // read each) and the X rows of every MFMA step.
      i32x2 qc[kFN];
#pragma unroll
      for (int j = 0; j < kFN; ++j) qc[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(TGEMM_LDS(i32x2, base + b_off[j]));
      bf16x8 fx[kSteps][MB];
#pragma unroll
      for (int u = 0; u < kSteps; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          fx[u][mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + x_rd[u] + mb * Sh::kXBlock));
      // Column block by column block; the conversions of block j+1 are
      // placed by hand between the MFMAs of block j and fenced there.  Left
      // to itself the compiler converted all blocks first and issued the
      // MFMAs in one burst (with both waves of a SIMD in step after each
      // barrier, one's conversions then rarely ran beside the other's
      // MFMAs): int8 5-6 % at 64 rows and up to 4 % at 1-32, int4 4-6 % at
      // 1-32 rows, bit-identical.  fw[j][u]: block j's bf16 operand of step u.
      u32x4 fw[kFN][kSteps];
      uint32_t hic[kFN][kSteps];
      constexpr int kParts = 4;  // conversion parts per block
      auto conv_part = [&](auto jc, auto pc) {
        constexpr int j = decltype(jc)::value, pp = decltype(pc)::value;
        if constexpr (BITS == 8) {
          fw[j][0][pp] = codes_pair_bf16<pp>(qc[j]);  // word pp of the one step
        } else {
          constexpr int u = pp / 2, h = pp % 2;  // step u, words 2h and 2h+1
          const uint32_t c = static_cast<uint32_t>(qc[j][u]);
          if constexpr (h == 0) hic[j][u] = c >> 4;
          const u32x2 w = nibble_words<h>(c, hic[j][u]);
          fw[j][u][2 * h] = w[0];
          fw[j][u][2 * h + 1] = w[1];
        }
      };
      static_for<kParts>([&](auto pc) { conv_part(std::integral_constant<int, 0>{}, pc); });
      constexpr int kPerBlock = kSteps * MB;  // MFMAs per column block
      static_for<kFN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        static_for<kPerBlock>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int u = i / MB, mb = i % MB;
          TGEMM_SCHED_FENCE();
          // kZeroStart: a group's first slice starts from zero.
          part[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fw[j][u]), fx[u][mb],
              (kZeroStart && kPos == 0 && u == 0) ? f32x4{} : part[mb][j], 0, 0, 0);
          if constexpr (j + 1 < kFN) {
            // Part pp of block j+1 after MFMA pp * kPerBlock / kParts of block j.
            static_for<kParts>([&](auto pc) {
              constexpr int pp = decltype(pc)::value;
              if constexpr (pp * kPerBlock / kParts == i) conv_part(std::integral_constant<int, j + 1>{}, pc);
            });
          }
        });
      });
      TGEMM_SCHED_FENCE();
      bool fold_now;
      if constexpr (kPos >= 0)
        fold_now = kPos == Sh::kSlicesPerGroup - 1 || t == te - 1;
      else
        fold_now = ((t % Sh::kSlicesPerGroup) == Sh::kSlicesPerGroup - 1 || t == te - 1) && (!kZeroStart || t < te);
      if (fold_now) {
        // End of a scale group: acc += s * partial, per column.
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
          f32x4 sc = *reinterpret_cast<const f32x4*>(base + s_rd + 64 * j);
          if constexpr (BITS == 4) sc *= kCodeScale;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][j][e] = __builtin_fmaf(part[mb][j][e], sc[e], acc[mb][j][e]);
            if constexpr (!kZeroStart) part[mb][j] = f32x4{};
          }
        }
      }
    };
    if constexpr (WqStages<BITS, MB, SPLIT>::kRegisters) {
      // R slices in flight per wave in registers; slice t goes to LDS
      // stage t % 2, its registers are refilled with slice t + R, and after
      // the barrier (stage t complete in every wave, stage t - 1 no longer
      // read) it is processed.
      constexpr int R = kRegSlices;
      auto step = [&](int t, WqRegs& r) {
        store_regs(t, r);
        load_regs(t + R, r);
        lds_barrier();
        process(t, t % NS, std::integral_constant<int, -1>{});
      };
      WqRegs r[R];
#pragma unroll
      for (int h = 0; h < R; ++h) load_regs(tb + h, r[h]);
      int t = tb;
      for (; t + R <= te; t += R) {
#pragma unroll
        for (int h = 0; h < R; ++h) step(t + h, r[h]);
      }
#pragma unroll
      for (int h = 0; h < R - 1; ++h)
        if (t + h < te) step(t + h, r[h]);
    } else {
      // kPerBar slices per barrier; their loads go kAhead slices ahead,
      // into the stages the previous group of slices occupied.
      constexpr int kPerBar = Sh::kPerBar;
      constexpr int kAhead = NS - kPerBar;
      // Slice tb + i lives in stage i % NS; the stages of the next issue
      // and the next process step along (a running count, not t % NS).
      for (int t = tb; t < tb + kAhead; ++t) issue_slice(t, t - tb);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - kPerBar) * kLoadsPerSlice) : "memory");
      lds_barrier();
      int si = kAhead, sp = 0;
      if constexpr (kZeroStart && kPerBar == 1) {
        // One scale group per iteration (ranges start on a group boundary),
        // so each slice's place in its group -- zero start, fold -- is known
        // at compile time and its conversions and MFMAs form one block of
        // straight-line code; only a partial last group checks te.
        constexpr int kSpg = Sh::kSlicesPerGroup;
        for (int t0 = tb; t0 < te; t0 += kSpg) {
          static_for<kSpg>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            const int t = t0 + u;
            if (u == 0 || t < te) {
              issue_slice(t + kAhead, si);
              si = si + 1 == NS ? 0 : si + 1;
              process(t, sp, std::integral_constant<int, u>{});
              sp = sp + 1 == NS ? 0 : sp + 1;
              asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - 1) * kLoadsPerSlice) : "memory");
              lds_barrier();  // the next slice landed everywhere; this one is no longer read
            }
          });
        }
      } else {
        for (int t = tb; t < te; t += kPerBar) {
#pragma unroll
          for (int h = 0; h < kPerBar; ++h) {
            issue_slice(t + kAhead + h, si);
            si = si + 1 == NS ? 0 : si + 1;
          }
#pragma unroll
          for (int h = 0; h < kPerBar; ++h) {
            process(t + h, sp, std::integral_constant<int, -1>{});
            sp = sp + 1 == NS ? 0 : sp + 1;
          }
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kAhead - kPerBar) * kLoadsPerSlice) : "memory");
          lds_barrier();  // the next slices landed everywhere; these are no longer read
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past K still land in LDS
    }
  }
}

// Epilogue: each lane holds 4 consecutive columns of one row per block.
template <int MB, int EPI, bool OUT_BF16>
__device__ __forceinline__ void wq_store(const W8Args& p, const f32x4 (&acc)[MB][kFN]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kBN;
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

template <int MB, int EPI, bool OUT_BF16, bool WHOLE>
__global__ __launch_bounds__(kThreads, 1) void tgemm_w8_thin(W8Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WqStages<8, MB>::kCount * WqShape<8>::kStage];
  f32x4 acc[MB][kFN];
  wq_accumulate<8, MB, WHOLE>(p, smem, acc);
  wq_store<MB, EPI, OUT_BF16>(p, acc);
}

template <int MB, int EPI, bool OUT_BF16, bool WHOLE>
__global__ __launch_bounds__(kThreads, 1) void tgemm_w4_thin(W8Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WqStages<4, MB>::kCount * WqShape<4>::kStage];
  f32x4 acc[MB][kFN];
  wq_accumulate<4, MB, WHOLE>(p, smem, acc);
  wq_store<MB, EPI, OUT_BF16>(p, acc);
}

// ---- Split-K for narrow weights.  With few 512-column stripes (a decode
// FFN projection, N of a few thousand) each compute unit streams at a few
// tens of GB/s and most units sit idle; the K range is then cut into
// chunks of whole scale groups (grid z).  Workgroup (stripe, z) writes its
// fp32 partial, already scaled group by group, to part[z][M][N]; the bf16
// thin kernel's reduction adds the partials in order of z, then the bias
// and the epilogue, and rounds once: deterministic, no atomics. ----
template <int BITS, int MB, bool WHOLE>
__global__ __launch_bounds__(kThreads, 1) void tgemm_wq_thin_splitk(W8Args p, float* part, int ktc) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WqStages<BITS, MB, true>::kCount * WqShape<BITS>::kStage];
  f32x4 acc[MB][kFN];
  const int KT = (p.K + WqShape<BITS>::kBK - 1) / WqShape<BITS>::kBK;
  const int tb = blockIdx.z * ktc;
  const int te = tb + ktc < KT ? tb + ktc : KT;
  wq_accumulate<BITS, MB, WHOLE, true>(p, smem, acc, tb, te);
  W8Args pp = p;
  pp.C = part + static_cast<int64_t>(blockIdx.z) * p.M * p.N;
  pp.ldc = p.N;
  pp.vec_c = (p.N % 4) == 0 ? 1 : 0;
  wq_store<MB, kEpiNone, false>(pp, acc);
}

// ---- The low-precision LM head with bias and LogSoftmax (the GEMM
// compute-cost page, section 7.2: its plan A, the integer weight, and plan
// B, the output projection, bias and LogSoftmax fused), pass 1: the stripe's
// logits with bias, their safe-softmax pair (row maximum m_w and
// s_w = sum exp(y - m_w) over the stripe) into part[row * G + w], and the
// fp32 logits into their buffer; pass 2 is the bf16 head's normalisation.
template <int BITS, int MB, bool WHOLE>
__global__ __launch_bounds__(kThreads, 1) void tgemm_wq_thin_lsm(W8Args p, LsmArgs q) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WqStages<BITS, MB>::kCount * WqShape<BITS>::kStage];
  f32x4 acc[MB][kFN];
  wq_accumulate<BITS, MB, WHOLE>(p, smem, acc);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kBN;
  constexpr int kWaves = kThreads / 64;
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
  // hold its columns; the eight waves meet in LDS.
  float* red = reinterpret_cast<float*>(smem);  // [8 waves][64 rows]
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
    float m = red[r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = __builtin_fmaxf(m, red[64 * w + r]);
    mrow[mb] = m;
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
      float srow = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) srow += red[64 * w + r];
      if (r < p.M) q.part[static_cast<int64_t>(r) * gridDim.x + blockIdx.x] = float2{mrow[mb], srow};
    }
  }

  // fp32 logits (bias already added) to their buffer.
  W8Args pl = p;
  pl.C = q.logits;
  pl.ldc = q.ldl;
  pl.vec_c = q.vec_l;
  wq_store<MB, kEpiNone, false>(pl, acc);
}

// Whether one buffer window can hold the widest stripe's bytes of Q (the
// first stripe's: rows 0 .. K-1 from column 0); X and the scales then fit
// too (X by wq_supported's row-stride bound, the scales being at most a
// sixteenth of Q's bytes).
bool wq_whole_window(int bits, const W8Args& a) {
  const int64_t rows = bits == 8 ? a.K : a.K / 2;
  return rows == 0 || (rows - 1) * a.ldq + a.N < (int64_t{1} << 31);
}

template <int BITS, int MB, int EPI, bool OUT_BF16>
hipError_t launch_m(const W8Args& a, hipStream_t s) {
  const dim3 grid((a.N + kBN - 1) / kBN);
  const bool whole = wq_whole_window(BITS, a);
  if constexpr (BITS == 8) {
    if (whole)
      hipLaunchKernelGGL((tgemm_w8_thin<MB, EPI, OUT_BF16, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((tgemm_w8_thin<MB, EPI, OUT_BF16, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (whole)
      hipLaunchKernelGGL((tgemm_w4_thin<MB, EPI, OUT_BF16, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((tgemm_w4_thin<MB, EPI, OUT_BF16, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int BITS, int MB>
hipError_t dispatch_epi(const W8Args& a, int epi, int out_bf16, hipStream_t s) {
  if (out_bf16) {
    if (epi == kEpiNone) return launch_m<BITS, MB, kEpiNone, true>(a, s);
    if (epi == kEpiBias) return launch_m<BITS, MB, kEpiBias, true>(a, s);
    return launch_m<BITS, MB, kEpiBiasGelu, true>(a, s);
  }
  if (epi == kEpiNone) return launch_m<BITS, MB, kEpiNone, false>(a, s);
  if (epi == kEpiBias) return launch_m<BITS, MB, kEpiBias, false>(a, s);
  return launch_m<BITS, MB, kEpiBiasGelu, false>(a, s);
}

template <int BITS>
hipError_t dispatch_m(const W8Args& a, int epi, int out_bf16, hipStream_t s) {
  if (a.M <= 16) return dispatch_epi<BITS, 1>(a, epi, out_bf16, s);
  if (a.M <= 32) return dispatch_epi<BITS, 2>(a, epi, out_bf16, s);
  if (a.M <= 48) return dispatch_epi<BITS, 3>(a, epi, out_bf16, s);
  return dispatch_epi<BITS, 4>(a, epi, out_bf16, s);
}

}  // namespace

bool wq_supported(int bits, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq) {
  // Whole 16-byte X chunks along K (K even, so int4 rows pair up), dword-
  // aligned Q rows (no dword of Q straddles a window end), per-lane offsets
  // below 2^31 (a slice's 32 byte rows of Q, 64 rows of X), and at most 64
  // rows.
  return (bits == 8 || bits == 4) && M <= 64 && K % 8 == 0 && N % 4 == 0 && ldq % 4 == 0 &&
         ldq * kRows < (int64_t{1} << 31) && ldx * 2 * 64 < (int64_t{1} << 31);
}

const char* wq_kernel_name(int bits, int M, bool split) {
  static const char* const kNames[2][4] = {
      {"tgemm_w8_thin_m16", "tgemm_w8_thin_m32", "tgemm_w8_thin_m48", "tgemm_w8_thin_m64"},
      {"tgemm_w4_thin_m16", "tgemm_w4_thin_m32", "tgemm_w4_thin_m48", "tgemm_w4_thin_m64"}};
  static const char* const kSplit[2][4] = {
      {"tgemm_w8_thin_splitk_m16+tgemm_splitk_reduce", "tgemm_w8_thin_splitk_m32+tgemm_splitk_reduce",
       "tgemm_w8_thin_splitk_m48+tgemm_splitk_reduce", "tgemm_w8_thin_splitk_m64+tgemm_splitk_reduce"},
      {"tgemm_w4_thin_splitk_m16+tgemm_splitk_reduce", "tgemm_w4_thin_splitk_m32+tgemm_splitk_reduce",
       "tgemm_w4_thin_splitk_m48+tgemm_splitk_reduce", "tgemm_w4_thin_splitk_m64+tgemm_splitk_reduce"}};
  const int m = M <= 16 ? 0 : M <= 32 ? 1 : M <= 48 ? 2 : 3;
  return (split ? kSplit : kNames)[bits == 8 ? 0 : 1][m];
}

hipError_t launch_wq_thin_lsm(int bits, const W8Args& a, const LsmArgs& q, int out_bf16,
                              hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(q.G));
  const int m = a.M <= 16 ? 1 : a.M <= 32 ? 2 : a.M <= 48 ? 3 : 4;
  const bool whole = wq_whole_window(bits, a);
#define TGEMM_WQ_LSM(B, MBV)                                                                          \
  do {                                                                                               \
    if (whole)                                                                                       \
      hipLaunchKernelGGL((tgemm_wq_thin_lsm<B, MBV, true>), grid, dim3(kThreads), 0, s, a, q);      \
    else                                                                                             \
      hipLaunchKernelGGL((tgemm_wq_thin_lsm<B, MBV, false>), grid, dim3(kThreads), 0, s, a, q);     \
  } while (0)
  if (bits == 8) {
    if (m == 1) TGEMM_WQ_LSM(8, 1);
    else if (m == 2) TGEMM_WQ_LSM(8, 2);
    else if (m == 3) TGEMM_WQ_LSM(8, 3);
    else TGEMM_WQ_LSM(8, 4);
  } else {
    if (m == 1) TGEMM_WQ_LSM(4, 1);
    else if (m == 2) TGEMM_WQ_LSM(4, 2);
    else if (m == 3) TGEMM_WQ_LSM(4, 3);
    else TGEMM_WQ_LSM(4, 4);
  }
#undef TGEMM_WQ_LSM
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lsm_normalize(q, a.C, a.ldc, a.M, a.N, a.vec_c, out_bf16, s);
}

ThinSplit wq_split_plan(int64_t M, int64_t N, int64_t K) {
  // Enough (stripe, chunk) workgroups to cover the compute units, chunks of
  // whole 128-row groups, and partial traffic (2 S M N fp32 = 8 S M N bytes)
  // at most half the int8 codes (K N bytes): S <= K / (16 M).  The plan does
  // not depend on the code width, so int4 and int8 codes of equal values sum
  // in the same order.
  ThinSplit r{1, 0};
  const int64_t stripes = (N + kBN - 1) / kBN;
  const int64_t G = (K + kGroupK - 1) / kGroupK;
  if (M < 1 || stripes > 128 || G < 2) return r;
  const int cus = device_cus();
  int64_t S = ((cus > 0 ? cus : 256) + stripes - 1) / stripes;
  S = S < G ? S : G;
  const int64_t cap = K / (16 * M);
  S = S < cap ? S : cap;
  if (S < 2) return r;
  const int64_t gpc = (G + S - 1) / S;  // groups per chunk
  r.S = static_cast<int>((G + gpc - 1) / gpc);
  r.ktc = static_cast<int>(gpc);  // in groups; the launcher converts to slices
  return r;
}

namespace {

template <int BITS, int MB>
hipError_t launch_splitk_bits_m(const W8Args& a, const ThinSplit& plan, float* part, hipStream_t s) {
  const int ktc = plan.ktc * WqShape<BITS>::kSlicesPerGroup;
  const dim3 grid((a.N + kBN - 1) / kBN, 1, plan.S);
  if (wq_whole_window(BITS, a))
    hipLaunchKernelGGL((tgemm_wq_thin_splitk<BITS, MB, true>), grid, dim3(kThreads), 0, s, a, part, ktc);
  else
    hipLaunchKernelGGL((tgemm_wq_thin_splitk<BITS, MB, false>), grid, dim3(kThreads), 0, s, a, part, ktc);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_splitk_bits(const W8Args& a, const ThinSplit& plan, float* part, hipStream_t s) {
  if (a.M <= 16) return launch_splitk_bits_m<BITS, 1>(a, plan, part, s);
  if (a.M <= 32) return launch_splitk_bits_m<BITS, 2>(a, plan, part, s);
  if (a.M <= 48) return launch_splitk_bits_m<BITS, 3>(a, plan, part, s);
  return launch_splitk_bits_m<BITS, 4>(a, plan, part, s);
}

}  // namespace

hipError_t launch_wq_thin(int bits, const W8Args& a, int epi, int out_bf16, hipStream_t s, float* part,
                          int64_t part_bytes) {
  if (part != nullptr) {
    const ThinSplit plan = wq_split_plan(a.M, a.N, a.K);
    if (plan.S > 1 && part_bytes >= thin_split_bytes(plan, a.M, a.N)) {
      hipError_t e = bits == 8 ? launch_splitk_bits<8>(a, plan, part, s) : launch_splitk_bits<4>(a, plan, part, s);
      if (e != hipSuccess) return e;
      Bf16Args r{};
      r.M = a.M;
      r.N = a.N;
      r.bias = a.bias;
      r.C = a.C;
      r.ldc = a.ldc;
      r.vec_c = a.vec_c;
      return launch_splitk_reduce(r, part, plan.S, epi, out_bf16, s);
    }
  }
  if (bits == 8) return dispatch_m<8>(a, epi, out_bf16, s);
  return dispatch_m<4>(a, epi, out_bf16, s);
}

}  // namespace tgemm
