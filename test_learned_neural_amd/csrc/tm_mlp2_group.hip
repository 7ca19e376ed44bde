// MFMA kernel for the 2-layer memory, d = 64, hidden = 256, chunk <= 64,
// bf16 keys/values/queries/outputs, fp32 state and gates: eight waves per
// workgroup, two per SIMD.
//
// Method ("Titans: Learning to Memorize at Test Time", mer.dev notes): the
// chunked test-time update of section 3.2 (gradients of every token of a
// chunk taken at the chunk-start weights), with the surprise momentum and
// forgetting of section 3.1, and retrieval after each token's write.  Per
// chunk of n tokens with chunk-start state (W_0, S_0):
//
//   a1  A_j = prod_{m<=j}(1-alpha_m), E_j = prod eta_m,
//       F_j = (1-alpha_j) F_{j-1} + E_j, U_i = theta_i prod_{m>i} eta_m,
//       D[j,i] = (1-alpha_j) D[j-1,i] + theta_i prod_{i<m<=j} eta_m (D[i,i] = theta_i)
//   a2  Z1 = K W1_0^T, A1 = SiLU(Z1), O = A1 W2_0^T
//   a3  Delta2 = O - V, Delta1 = (Delta2 W2_0) * SiLU'(Z1)
//   a5  Zq1 = diag(A) Q W1_0^T + diag(F) Q S1_0^T - (D o Q K^T) Delta1, H1 = SiLU(Zq1)
//       y   = diag(A) H1 W2_0^T + diag(F) H1 S2_0^T - (D o H1 A1^T) Delta2
//   a4  W_l <- A_n W_l + F_n S_l - G_l(D[n-1,:]),  S_l <- E_n S_l - G_l(U)
//       G_1(w) = sum_j w_j Delta1_j k_j^T,  G_2(w) = sum_j w_j Delta2_j a1_j^T
//
// MI355X mapping
// --------------
// * Each (batch, head) stream runs on a PAIR of workgroups (two CUs), one per
//   half of the hidden layer.  A workgroup is eight waves, two per SIMD, and
//   wave w owns 16 hidden units: its share of the state (W1, S1, W2, S2
//   restricted to those units, 64 floats per lane) lives in ordinary VGPRs
//   for the whole sequence, in the accumulator layout of
//   v_mfma_f32_16x16x32_f16 with rows = the d index and lanes = the units.
//   Such a tile is, without any move, the MFMA operand of every product that
//   contracts over d (Z1, Zq1, Delta1), and the weighted outer-product folds
//   (G_1, G_2) land in that same layout.
// * Products that contract over the tokens of the chunk (the folds, the
//   masked first-layer term) take the per-wave activations straight from
//   their accumulators (lanes = units, registers = tokens).
// * Products that contract over the hidden units (O, the masked scores
//   H1 A1^T, y) run once per workgroup: every wave writes its A1, H1 and
//   W2/S2 pieces to LDS; O and the scores are two 16x16 output tiles per
//   wave over all 128 units of the workgroup, y four 32x32 blocks on waves
//   0..3 (one per SIMD).  Only O (needed before the backprop: one
//   exchange per chunk on the critical path) and y (exchanged one chunk late,
//   riding on the next O exchange) cross the pair, as partial sums.
// * A tile used by products that contract over either of its dimensions is
//   stored once in LDS, K-major for one use (a lane's four accumulator rows
//   are one 8-byte store), and read along its other dimension with the
//   transposing ds_read_b64_tr_b16 (see tr4).
// * The second wave per SIMD fills the issue gaps of the first: the
//   element-wise work (SiLU, its derivative, scaling, conversions) and the
//   barriers of one wave overlap the matrix work of the other.
// * Every MFMA operand is fp16 with a power-of-two scale per operand block
//   and chunk (fp32 accumulation, exact rescaling): the state, the
//   activations and the residuals (A1 and H1, computed in units of -1/ln 2
//   for their SiLUs, are converted back by their fp16 conversion factor).
//   Scores produced by one wave and consumed
//   in one K-step carry that wave's own scale, so they need no workgroup-wide
//   maximum.
// * The pair exchanges its partial sums through global memory in 8-byte
//   words that carry the chunk's sequence number beside the value (single-
//   copy-atomic 64-bit agent-coherent stores): each reader polls its own
//   words until they carry the number it expects, so the exchange needs no
//   flag, no wait for store completion and no barrier around the wait.  A
//   formal release/acquire flag protocol at agent scope costs an L2
//   writeback and invalidation per chunk (measured 3.5 -> 4.4 ms per call on
//   the earlier four-wave kernel).  The coefficient scan and the products
//   that need no partner data run while the exchange is in flight.  A
//   thread whose partner's words do not arrive within a bounded spin gives
//   up: the workgroup records the failure in the workspace status word
//   (returned by titans_mem_workspace_status) and writes NaN to W_out, S_out
//   and y of every stream the pair serves.  Sums are formed in a fixed order
//   (half 0 + half 1), so results are bitwise reproducible and identical in
//   both halves.
// * With few streams (at most a quarter as many as CUs) each half's
//   retrieval runs on a workgroup of its own, one chunk behind (kSplit):
//   the key-side workgroup hands it the chunk-start W2/S2 copies, A1, Delta2,
//   Delta1 and the query products in the same tagged words, and the
//   retrieval workgroup computes the masked scores, H1 and y.  A stream
//   then keeps four CUs busy, and each side's chunk is the shorter for it.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

namespace titans {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kD = 64;
constexpr int kH = 256;
constexpr int kB = 64;               // token rows per chunk tile
constexpr int kUW = 16;              // hidden units per wave
constexpr int kMaxWaves = 8;         // per-wave LDS slots and stage stamps
constexpr int kP = 2 * kD * kH;
constexpr int RS = 72;               // fp16 row stride (halves) of 64-wide tiles: 144-byte rows
constexpr int RF = 68;               // fp32 row stride of D
constexpr unsigned kSpinMax = 1u << 21;

// ---- LDS layout (bytes): the part common to both workgroup sizes ----
constexpr int kT64 = kB * RS * 2;    // 9216
constexpr int OFF_K = 0;             // K   [j][c]
constexpr int OFF_Q = OFF_K + kT64;      // Q   [j][c]
constexpr int OFF_YP = OFF_Q + kT64;     // y partials parked across the chunk boundary (fp32)
constexpr int OFF_D2T = OFF_YP + kT64;   // Delta2^T [c][j]
constexpr int OFF_SC = OFF_D2T + kT64;   // masked scores [i][j] (keys i, queries j): first layer, then second
constexpr int OFF_DM = OFF_SC + kT64;    // D [j][i] fp32
// coefficient area (relative offsets)
// float index: XT = the D recurrences' carried products at rows 31 and 63
// (see the a1 stage), T11/T12 = transfer of rows 32..63 (32 entries each)
constexpr int COEF_XT = 0, COEF_T11 = 64, COEF_T12 = 96, COEF_THETA = 128, COEF_A = 192, COEF_E = 256,
              COEF_F = 320;
constexpr int COEF_H16 = 384 * 4;                                   // byte offset of fp16 arrays
constexpr int H16_WU = 0, H16_WD = 64;                              // half index: the fold weights
constexpr int COEF_INT = COEF_H16 + 128 * 2;                        // byte offset of int slots
constexpr int COEF_PAIR = COEF_INT + 64 * 4;                        // byte offset of (1-alpha, eta) pairs
constexpr int kCoefBytes = COEF_PAIR + kB * 8;
// staging for the next chunk's raw bf16 K, Q rows (row-major, 128 bytes a
// row) and gates, filled one chunk ahead with LDS-direct loads
constexpr int kStageBytes = 2 * kB * kD * 2 + 3 * kB * 4;

// ---- the workgroup size: NW waves of 16 hidden units, 256 / (16 NW) workgroups per stream ----
// The library uses NW = 8 (two workgroups per stream, two waves per SIMD);
// the layout and the kernel are written for any NW that divides 16 with
// NW >= 4, the group exchange for any number of workgroups per stream.
template <int NW>
struct Grp {
  static constexpr int kWaves = NW;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kUG = kUW * NW;          // hidden units per workgroup
  static constexpr int kG = kH / kUG;           // workgroups per stream
  static constexpr int kT = 16 / NW;            // 16x16 tiles per wave of a 64x64 workgroup product
  static constexpr int kE = 4 * kT;             // values per thread of such a product
  static constexpr int kYRows = kB / kG;        // y rows (tokens) of a chunk one workgroup finishes
  static constexpr int kYElems = kYRows * kD;   // ... as elements
  static constexpr int kYPer = kYElems / kThreads;   // ... per thread
  static constexpr int kKSteps = kUG / 32;      // K-steps of a product over the workgroup's units
  static constexpr int kRowPasses = 512 / kThreads;   // 16-byte row pieces of a chunk tile per thread
  static constexpr int kTU = kUG * RS * 2;
  static constexpr int OFF_A1 = OFF_DM + kB * RF * 4;   // A1^T [u][j] over the workgroup's units
  static constexpr int OFF_H1 = OFF_A1 + kTU;           // H1^T [u][j]
  static constexpr int OFF_W2 = OFF_H1 + kTU;           // W2^T [u][c]
  static constexpr int OFF_S2 = OFF_W2 + kTU;           // S2^T [u][c]
  static constexpr int OFF_COEF = OFF_S2 + kTU;
  static constexpr int OFF_STAGE = (OFF_COEF + kCoefBytes + 255) / 256 * 256;
  static constexpr int kLdsBytes = OFF_STAGE + kStageBytes;
  // waves that run the coefficient recurrences during the exchange: D rows
  // 0..31, D rows 32..63 (and the fold weights), the scans
  static constexpr int kWD0 = NW == 8 ? 3 : 1, kWD1 = NW == 8 ? 5 : 2, kWS = NW == 8 ? 6 : 3;
  // exchange words per group: O partials [workgroup][parity][word e][thread]
  // and y partials [sender][receiver slot][parity][element of the receiver's rows]
  static constexpr int64_t kXOWords = (int64_t)kG * 2 * kThreads * (kE / 2);   // two values a word
  static constexpr int64_t kXYWords = (int64_t)kG * (kG - 1) * 2 * (kYElems / 2);
  static constexpr int64_t kGroupBytes = (kXOWords + kXYWords) * 8;
  static constexpr int kMaxGroups = 256 / kG;   // one workgroup per CU of a 256-CU device
  // few-stream split (kSplit): the words a key-side workgroup hands its
  // retrieval workgroup per thread and chunk ([half][parity][word][thread]),
  // written at three points of the chunk: the chunk-start W2 and S2 copies
  // and A1 (words PW_1 ..), Delta2 and the query products (PW_2 ..), Delta1
  // (PW_3 ..); and the retrieval workgroups' receipts ([half][thread])
  static constexpr int kPubW = 34;
  static constexpr int PW_1 = 0, PW_2 = 17, PW_3 = 28;
  static constexpr int64_t kXPWords = (int64_t)kG * 2 * kPubW * kThreads;
  static constexpr int64_t kXAWords = (int64_t)kG * kThreads;
  static constexpr int64_t kGroupBytesSplit = kGroupBytes + (kXPWords + kXAWords) * 8;
  static constexpr int kMaxGroupsSplit = 256 / (2 * kG);
  static_assert(NW == 8 || NW == 4, "eight or four waves");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kYElems * 4 <= kT64, "the parked y tiles fit their area");
  static_assert(kYPer * kThreads == kYElems && kYPer % 2 == 0, "every thread finishes the same number of y rows pairs");
};

// int slots
constexpr int INT_AMAX_D2 = 0, INT_EWU = 1, INT_EWD = 2, INT_FAIL = 3, INT_T22 = 4;
constexpr int INT_M2 = 8;     // per-wave maxima of |W2|, |S2| (8 slots)
// (the state's slots M1, M2, N1 are written by the fold of the previous
// chunk, or at the stream's start, and read after the next chunk's first
// barrier: no per-lane value is carried across the chunk boundary)
constexpr int INT_N1 = 16;    // per-wave maxima of |W1| (a bound on the A1 scale)
constexpr int INT_MH1 = 24;   // per-wave maxima of |H1| log2 e
constexpr int INT_ESC = 32;   // per-wave exponents of the first-layer masked scores
constexpr int INT_EDP = 40;   // per-wave exponents of the second-layer masked scores
constexpr int INT_NK = 48;    // per-wave maxima of |K|
constexpr int INT_M1 = 56;    // per-wave maxima of |W1|, |S1| (each wave's own operand scale)

// Exchange words are 8 bytes: two values and the low bits of the sequence
// number of the chunk that wrote them (see tstore / tpoll).

// ---- stage timing (a build option; off in the library) ----
// With TM_STAGE_STAMPS=1 the eight waves of the first key-side workgroup
// (with TM_STAMP_R=1 as well: of the first retrieval workgroup of a split
// launch) record the shader clock (s_memtime) at every stage boundary of
// chunks kStampFrom .. kStampFrom + kStampChunks - 1 of its first stream;
// titans_mem_stage_stamps (exported by that build only) copies them out.
// stage_stamps.py builds the instrumented library and prints the per-stage
// table.
#ifndef TM_STAGE_STAMPS
#define TM_STAGE_STAMPS 0
#endif
#ifndef TM_STAMP_R
#define TM_STAMP_R 0
#endif
constexpr int kStampStages = 24, kStampFrom = 16, kStampChunks = 64;
#if TM_STAGE_STAMPS
__device__ unsigned long long stage_stamps[kStampChunks * kMaxWaves * kStampStages];
#define STAMP(k)                                                                                       \
  do {                                                                                                 \
    if (stamp_slot >= 0 && lane == 0)                                                                  \
      stage_stamps[(stamp_slot * kMaxWaves + w) * kStampStages + (k)] = __builtin_amdgcn_s_memtime();  \
  } while (0)
#else
#define STAMP(k) \
  do {           \
  } while (0)
#endif

struct Params {
  int N, chunk, streams, n_groups;
  const __hip_bfloat16* k;
  const __hip_bfloat16* v;
  const __hip_bfloat16* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  const float* W_in;
  const float* S_in;
  __hip_bfloat16* y;
  float* W_out;
  float* S_out;
  unsigned char* xbuf;   // n_groups * Grp<NW>::kGroupBytes, zeroed before every launch
  unsigned* status;      // set to 1 when a group gave up waiting
  unsigned spin_max;
  int chunk_gates;       // gates hold one value per chunk
  int gstride;           // gates per stream: N, or ceil(N / chunk) with per-chunk gates
};

// index of the gate of the first token of chunk ci (token c0) of stream s
__device__ __forceinline__ int64_t gate_base(const Params& p, int s, int ci, int c0) {
  return (int64_t)s * p.gstride + (p.chunk_gates ? ci : c0);
}

__device__ __forceinline__ f4v mfma(h8 a, h8 b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
typedef float f16v __attribute__((ext_vector_type(16)));
// v_mfma_f32_32x32x16_f16: lane l serves row (A) or column (B) l % 32 with
// K values 8 (l / 32) .. + 7; accumulator register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
__device__ __forceinline__ f16v mfma32(h8 a, h8 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// x f rounded to fp16 as a multiply and a conversion (two values share one
// v_cvt_pk_f16_f32).  The empty asm keeps the compiler from fusing the pair
// into v_fma_mix, which issues more slowly on this hardware.
__device__ __forceinline__ _Float16 sc16(float x, float f) {
  float y = x * f;
  asm("" : "+v"(y));
  return (_Float16)y;
}

// Operand fragments of v_mfma_f32_16x16x32_f16.  Lane l serves row (A) or
// column (B) l & 15 and K group g = l >> 4 with 8 values.  Two orders of the
// K slots are used (any order works if both operands of a product agree):
// * register order, for products with an operand taken from accumulator
//   tiles: slot i < 4 is k = kb + 4g + i, slot i >= 4 is k = kb + 16 + 4g +
//   i - 4, i.e. rows 4g + i of two consecutive 16-row tiles;
// * consecutive order, for products with both operands in LDS: slot i is
//   k = kb + 8g + i (one 16-byte read).
__device__ __forceinline__ h8 frag_rk(const _Float16* row, int kb, int g) {
  const h4 lo = *(const h4*)(row + kb + 4 * g);
  const h4 hi = *(const h4*)(row + kb + 16 + 4 * g);
  return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ h8 frag_c8(const _Float16* row, int kb, int g) {
  return *(const h8*)(row + kb + 8 * g);
}
// two accumulator tiles (rows 0-15 and 16-31 of a K block) as a
// register-order fragment, scaled to fp16
__device__ __forceinline__ h8 tiles_frag(const f4v a, const f4v b, float f) {
  return h8{sc16(a[0], f), sc16(a[1], f), sc16(a[2], f), sc16(a[3], f),
            sc16(b[0], f), sc16(b[1], f), sc16(b[2], f), sc16(b[3], f)};
}

// Transposing fp16 reads from LDS (ds_read_b64_tr_b16).  The 16 lanes of
// K group g read a 4 x 16 block of a row-major tile T (row stride S halves):
// rows k0 .. k0 + 3, columns n0 .. n0 + 15, k0 the same for the group; lane
// (g, lc) receives column n0 + lc of the four rows.  Lane j of a group
// supplies the address of row k0 + j / 4, columns n0 + 4 (j % 4) .. + 3: the
// instruction hands element e of lane i the (i % 4)-th value read by lane
// 4e + i / 4 of its group (lane layout measured on gfx950).  Tiles consumed
// with K along both of their dimensions are stored once, K-major, with one
// 8-byte store per accumulator tile and lane (its four consecutive rows),
// and read along the other dimension with these reads.
__device__ __forceinline__ h4 tr4(const _Float16* T, int S, int k0, int n0, int lc) {
  typedef __fp16 fp16x4 __attribute__((vector_size(8)));
  typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;
  return __builtin_bit_cast(
      h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(T + (k0 + (lc >> 2)) * S + n0 + 4 * (lc & 3))));
}
// operand fragment of row / column n0 + lc from a K-major tile: register
// order (frag_rk) and consecutive order (frag_c8) of the K slots
__device__ __forceinline__ h8 frag_tr_rk(const _Float16* T, int S, int kb, int n0, int g, int lc) {
  const h4 lo = tr4(T, S, kb + 4 * g, n0, lc), hi = tr4(T, S, kb + 16 + 4 * g, n0, lc);
  return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ h8 frag_tr_c8(const _Float16* T, int S, int kb, int n0, int g, int lc) {
  const h4 lo = tr4(T, S, kb + 8 * g, n0, lc), hi = tr4(T, S, kb + 8 * g + 4, n0, lc);
  return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// the four consecutive rows of a lane's accumulator tile, stored K-major:
// row `row` of T, columns col0 .. col0 + 3
__device__ __forceinline__ void store_rows4(_Float16* T, int S, int row, int col0, h4 v) {
  *(h4*)(T + row * S + col0) = v;
}
__device__ __forceinline__ h4 to_h4(const f4v v, float f) {
  return h4{sc16(v[0], f), sc16(v[1], f), sc16(v[2], f), sc16(v[3], f)};
}

// ---- cross-lane helpers on DPP (no LDS traffic); call with all 64 lanes active ----
// DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_shr:n = 0x110 + n,
// row_mirror = 0x140, row_half_mirror = 0x141, row_bcast:15 = 0x142, row_bcast:31 = 0x143
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, false));
}
// lanes whose DPP source is out of range (or whose row is masked off) get `ident`
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp_or(float ident, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(x), kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// maximum over the wave, returned uniformly: the rows of 16 lanes reduce
// among themselves, then rows 1 and 3 take in rows 0 and 2 (row_bcast:15)
// and rows 2 and 3 take in the maximum of rows 0 and 1 (row_bcast:31), so
// lane 63 ends with the wave's maximum (one lane read instead of four)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));   // every lane of a row of 16 holds the row's maximum
  v = fmaxf(v, dpp_or<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_or<0x143, 0xc>(v, v));
  return lane_value(v, 63);
}

// inclusive prefix product over the lanes (lane l: x_0 * ... * x_l)
__device__ __forceinline__ float wave_prefix_prod(float x) {
  x *= dpp_or<0x111>(1.f, x);
  x *= dpp_or<0x112>(1.f, x);
  x *= dpp_or<0x114>(1.f, x);
  x *= dpp_or<0x118>(1.f, x);
  x *= dpp_or<0x142, 0xa>(1.f, x);
  x *= dpp_or<0x143, 0xc>(1.f, x);
  return x;
}

// inclusive scan of the affine maps f_l(u) = a_l u + b_l over the lanes:
// on return lane l holds f_l o ... o f_0 as (a, b), i.e. a = a_0 ... a_l and
// b = the value of u_l = a_l u_{l-1} + b_l started from u_{-1} = 0
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ void affine_step(float& a, float& b) {
  const float a2 = dpp_or<kCtrl, kRowMask>(1.f, a);
  const float b2 = dpp_or<kCtrl, kRowMask>(0.f, b);
  b = fmaf(a, b2, b);
  a *= a2;
}
__device__ __forceinline__ void wave_affine_scan(float& a, float& b) {
  affine_step<0x111>(a, b);
  affine_step<0x112>(a, b);
  affine_step<0x114>(a, b);
  affine_step<0x118>(a, b);
  affine_step<0x142, 0xa>(a, b);
  affine_step<0x143, 0xc>(a, b);
}

// power-of-two scale exponent bringing amax into [2^13, 2^14)
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 0;
  int e;
  (void)frexpf(amax, &e);
  return 14 - e;
}
// 2^-k as a float multiplier: exact rescaling while 2^-k is a normal float,
// i.e. k <= 126; beyond that the factor flushes towards zero (scaled values
// far below any tolerance floor).  k is clamped below so that the factor
// stays finite.
__device__ __forceinline__ float pow2neg(int k) { return ldexpf(1.f, -max(k, -126)); }
// 2^e as a float multiplier for the scalings up to fp16 operands (one
// multiply per element instead of an ldexp; computed once per block).  Equal
// to ldexpf(x, e) whenever e <= 127, i.e. unless the block's amax is below
// 2^-113, where the clamped scale leaves the operand smaller than [2^13, 2^14)
// but still far below every tolerance floor.
__device__ __forceinline__ float pow2pos(int e) { return ldexpf(1.f, min(e, 127)); }

// The SiLUs take their argument in units of -1/ln 2 (x = -z log2 e, folded
// into the scale that unscales z), so that sigmoid(z) = 1 / (1 + 2^x) needs
// no multiply before the exponential.
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float sigmoid_x(float x) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x)); }

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ h8 bf16x8_to_h8(uint4 u) {
  return h8{(_Float16)bf16_lo(u.x), (_Float16)bf16_hi(u.x), (_Float16)bf16_lo(u.y), (_Float16)bf16_hi(u.y),
            (_Float16)bf16_lo(u.z), (_Float16)bf16_hi(u.z), (_Float16)bf16_lo(u.w), (_Float16)bf16_hi(u.w)};
}

// Group exchange: every 8-byte word carries two values and the low 8 bits
// of the sequence number of the chunk that wrote them, stored with one
// single-copy-atomic 64-bit agent-coherent (sc1) store.  A reader polls its
// own words until each carries the tag it expects, so no flag,
// store-completion wait or barrier orders the exchange: a word is either
// the old one (old tag) or the new one, never a mix.  A value keeps the
// sign, the exponent and the 19 leading mantissa bits of its fp32 form
// (truncated: a relative error below 2^-19, far under the fp16 rounding the
// exchanged sums go through next).  Two parities double-buffer the chunks,
// so a slot holds the words of chunk seq - 2 (tag seq - 2, distinct from
// seq mod 256) until it is rewritten; sequence numbers start at 1 and the
// buffers are zeroed before every launch, and by the first chunk whose tag
// is 0 (seq = 256) every slot has been written, so no word of an earlier
// call or an unwritten slot can match.  The buffers are thread-major: word
// e of thread t sits at e * stride + t, so each store or load instruction
// of a wave covers 512 contiguous bytes (whole lines: an agent-coherent
// store writes through L2), and a partner's thread reads back exactly the
// words the same thread wrote.  A partner overwrites a slot two chunks
// later, after having read this workgroup's next chunk, which this
// workgroup writes only after reading the slot.
__device__ __forceinline__ unsigned long long tword(float v0, float v1, unsigned tag) {
  return ((unsigned long long)(tag & 0xffu) << 56) | ((unsigned long long)(__float_as_uint(v1) >> 4) << 28) |
         (unsigned long long)(__float_as_uint(v0) >> 4);
}
__device__ __forceinline__ void tstore(unsigned long long* base, int idx, float v0, float v1, unsigned tag) {
  __hip_atomic_store(base + idx, tword(v0, v1, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// words t, t + kStride, ..., t + (kW - 1) kStride of each of the kN bases,
// until all carry `tag` (the loads of all bases are in flight together);
// word e holds values 2e and 2e + 1 of out[b].  false = gave up after
// spin_max polls (spin_max = 0 gives up at once: the failure-path test hook)
template <int kStride, int kW, int kN>
__device__ __forceinline__ bool tpoll(const unsigned long long* const (&base)[kN], int t, unsigned tag,
                                      unsigned spin_max, float (&out)[kN][2 * kW]) {
  for (unsigned it = 0; it < spin_max; ++it) {
    unsigned long long wd[kN][kW];
#pragma unroll
    for (int b = 0; b < kN; ++b)
#pragma unroll
      for (int e = 0; e < kW; ++e)
        wd[b][e] = __hip_atomic_load(base[b] + (e * kStride + t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int b = 0; b < kN; ++b)
#pragma unroll
      for (int e = 0; e < kW; ++e) {
        out[b][2 * e] = __uint_as_float((unsigned)(wd[b][e] & 0x0fffffffu) << 4);
        out[b][2 * e + 1] = __uint_as_float((unsigned)((wd[b][e] >> 28) & 0x0fffffffu) << 4);
        ok = ok && (unsigned)(wd[b][e] >> 56) == (tag & 0xffu);
      }
    if (ok) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// tpoll's first round issued early: the loads go out at once, the tags are
// checked later (check), and only a miss falls back to tpoll
template <int kStride, int kW, int kN>
struct TPollEarly {
  unsigned long long wd[kN][kW];
  __device__ __forceinline__ void issue(const unsigned long long* const (&base)[kN], int t) {
#pragma unroll
    for (int b = 0; b < kN; ++b)
#pragma unroll
      for (int e = 0; e < kW; ++e)
        wd[b][e] = __hip_atomic_load(base[b] + (e * kStride + t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ bool check(unsigned tag, float (&out)[kN][2 * kW]) const {
    bool ok = true;
#pragma unroll
    for (int b = 0; b < kN; ++b)
#pragma unroll
      for (int e = 0; e < kW; ++e) {
        out[b][2 * e] = __uint_as_float((unsigned)(wd[b][e] & 0x0fffffffu) << 4);
        out[b][2 * e + 1] = __uint_as_float((unsigned)((wd[b][e] >> 28) & 0x0fffffffu) << 4);
        ok = ok && (unsigned)(wd[b][e] >> 56) == (tag & 0xffu);
      }
    return ok;
  }
};

// Hand-over words (few-stream split, see kSplit): the same single-copy-
// atomic tagged 8-byte words as the exchange above, carrying either three
// 16-bit values (fp16 operands, or an operand's scale exponent as a 16-bit
// integer, which can exceed 8 bits for values near fp32's underflow) and the
// tag, or two truncated fp32 values and the tag (tword).
__device__ __forceinline__ unsigned long long h3word(unsigned short a, unsigned short b, unsigned short c,
                                                     unsigned tag) {
  return (unsigned long long)a | ((unsigned long long)b << 16) | ((unsigned long long)c << 32) |
         ((unsigned long long)(tag & 0xffu) << 56);
}
__device__ __forceinline__ unsigned short hbits(_Float16 x) { return __builtin_bit_cast(unsigned short, x); }
__device__ __forceinline__ unsigned short ebits(int e) { return (unsigned short)(short)e; }
__device__ __forceinline__ _Float16 h3_get(unsigned long long wd, int k) {
  return __builtin_bit_cast(_Float16, (unsigned short)(wd >> (16 * k)));
}
__device__ __forceinline__ int h3_int(unsigned long long wd, int k) { return (int)(short)(unsigned short)(wd >> (16 * k)); }
__device__ __forceinline__ float tword_lo(unsigned long long wd) { return __uint_as_float((unsigned)(wd & 0x0fffffffu) << 4); }
__device__ __forceinline__ float tword_hi(unsigned long long wd) {
  return __uint_as_float((unsigned)((wd >> 28) & 0x0fffffffu) << 4);
}
__device__ __forceinline__ bool tag_is(unsigned long long wd, unsigned tag) { return (unsigned)(wd >> 56) == (tag & 0xffu); }
__device__ __forceinline__ void wstore(unsigned long long* p, unsigned long long wd) {
  __hip_atomic_store(p, wd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// kW words of one thread (word e at e * kStride + t): the loads of a range
// of them issued together, the range's tags checked later, and the range
// reloaded until they match
template <int kStride, int kW>
struct TagWords {
  unsigned long long wd[kW];
  template <int kLo, int kHi>
  __device__ __forceinline__ void issue(const unsigned long long* base, int t) {
#pragma unroll
    for (int e = kLo; e < kHi; ++e)
      wd[e] = __hip_atomic_load(base + (e * kStride + t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  template <int kLo, int kHi>
  __device__ __forceinline__ bool ok(unsigned tag) const {
    bool r = true;
#pragma unroll
    for (int e = kLo; e < kHi; ++e) r = r && tag_is(wd[e], tag);
    return r;
  }
  // false = gave up after spin_max polls
  template <int kLo, int kHi>
  __device__ __forceinline__ bool wait(const unsigned long long* base, int t, unsigned tag, unsigned spin_max) {
    if (ok<kLo, kHi>(tag)) return true;
    for (unsigned it = 0; it < spin_max; ++it) {
      __builtin_amdgcn_s_sleep(1);
      issue<kLo, kHi>(base, t);
      if (ok<kLo, kHi>(tag)) return true;
    }
    return false;
  }
};

// A chunk's raw inputs, one thread's share: for each of its row pieces
// (piece = tid + r * kThreads, r < 512 / kThreads) 16 bytes (8 bf16) of row
// j = piece / 8 of K and of Q (columns 8 (piece % 8) ..), and for tid < 64
// the gates of token tid.  Rows and tokens past the chunk end read as zeros
// (gates as "no forgetting, no decay, no write").
template <int kPasses>
struct ChunkRegs {
  uint4 k[kPasses], q[kPasses];
  float ga, ge, gt;
};

template <int kThreads>
__device__ __forceinline__ ChunkRegs<512 / kThreads> load_chunk_regs(const Params& p, int64_t row0, int64_t g0,
                                                                      int n, int tid) {
  ChunkRegs<512 / kThreads> r;
#pragma unroll
  for (int rr = 0; rr < 512 / kThreads; ++rr) {
    const int piece = tid + rr * kThreads, j = piece >> 3, cb = (piece & 7) * 8;
    if (j < n) {
      r.k[rr] = *(const uint4*)(p.k + (row0 + j) * kD + cb);
      r.q[rr] = *(const uint4*)(p.q + (row0 + j) * kD + cb);
    } else {
      r.k[rr] = r.q[rr] = make_uint4(0, 0, 0, 0);
    }
  }
  r.ga = 0.f; r.ge = 1.f; r.gt = 0.f;
  if (tid < kB && tid < n) {
    const int64_t gi = g0 + (p.chunk_gates ? 0 : tid);
    r.ga = p.alpha[gi];
    r.ge = p.eta[gi];
    r.gt = p.theta[gi];
  }
  return r;
}

// Prefetch of a chunk's raw rows straight into the LDS staging area
// (global_load_lds: lane l of an instruction writes 16 bytes at base + 16 l,
// or 4 bytes at base + 4 l; lanes that do not load write nothing).  Piece
// `piece` of load_chunk_regs goes to slot `piece` of each area, so the area
// holds the chunk's rows in row-major order and each thread later reads back
// what it loaded itself.  Wave 0 loads the gates.  Rows and tokens past the
// chunk end are left out and replaced on unstaging.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
template <int kThreads>
__device__ __forceinline__ void prefetch_chunk_lds(const Params& p, int64_t row0, int64_t g0, int n, int tid,
                                                   unsigned char* stage) {
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  uint4* sk = (uint4*)stage;
  uint4* sq = (uint4*)(stage + kB * kD * 2);
#pragma unroll
  for (int rr = 0; rr < 512 / kThreads; ++rr) {
    const int piece = tid + rr * kThreads, j = piece >> 3, cb = (piece & 7) * 8;
    const int slot = 64 * (w + rr * (kThreads / 64));
    if (j < n) {
      __builtin_amdgcn_global_load_lds((const void*)(p.k + (row0 + j) * kD + cb), (lds_void_ptr)(sk + slot), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(p.q + (row0 + j) * kD + cb), (lds_void_ptr)(sq + slot), 16, 0, 0);
    }
  }
  if (w == 0 && lane < n) {
    float* g = (float*)(stage + 2 * kB * kD * 2);
    const int64_t gi = g0 + (p.chunk_gates ? 0 : lane);   // per-chunk gates: every lane loads the one value
    __builtin_amdgcn_global_load_lds((const void*)(p.alpha + gi), (lds_void_ptr)g, 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(p.eta + gi), (lds_void_ptr)(g + kB), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(p.theta + gi), (lds_void_ptr)(g + 2 * kB), 4, 0, 0);
  }
}

template <int kThreads>
__device__ __forceinline__ ChunkRegs<512 / kThreads> unstage_chunk_regs(const unsigned char* stage, int n, int tid) {
  ChunkRegs<512 / kThreads> r;
#pragma unroll
  for (int rr = 0; rr < 512 / kThreads; ++rr) {
    const int piece = tid + rr * kThreads;
    if ((piece >> 3) < n) {
      r.k[rr] = ((const uint4*)stage)[piece];
      r.q[rr] = ((const uint4*)(stage + kB * kD * 2))[piece];
    } else {
      r.k[rr] = r.q[rr] = make_uint4(0, 0, 0, 0);
    }
  }
  r.ga = 0.f; r.ge = 1.f; r.gt = 0.f;
  if (tid < kB && tid < n) {
    const float* g = (const float*)(stage + 2 * kB * kD * 2);
    r.ga = g[tid]; r.ge = g[kB + tid]; r.gt = g[2 * kB + tid];
  }
  return r;
}

// the exchange buffers (no word may carry a valid sequence number) and the
// status word, cleared before every launch by a fill kernel
__global__ void zero_exchange_kernel(uint4* buf, int64_t n16, unsigned* status) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    buf[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
}

// A workgroup that gave up waiting for a partner writes NaN to W_out, S_out
// and y of every stream its group serves (s = group, group + n_groups, ...),
// after all of its own earlier writes, so a give-up never passes for a
// result, in place or not.  The partners give up as well at their next wait
// and do the same; only a partner that had already passed its last wait
// can still write rows of its own afterwards.
template <int kThreads>
__device__ void poison_group_streams(const Params& p, int grp, int tid) {
  const unsigned fnan = __float_as_uint(__builtin_nanf(""));
  const uint4 f4 = make_uint4(fnan, fnan, fnan, fnan);
  const uint4 b8 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);   // bf16 quiet NaNs
  for (int s = grp; s < p.streams; s += p.n_groups) {
    uint4* Wo = (uint4*)(p.W_out + (int64_t)s * kP);
    uint4* So = (uint4*)(p.S_out + (int64_t)s * kP);
    for (int i = tid; i < kP / 4; i += kThreads) {
      Wo[i] = f4;
      So[i] = f4;
    }
    uint4* yo = (uint4*)(p.y + (int64_t)s * p.N * kD);
    const int64_t ny = (int64_t)p.N * kD / 8;
    for (int64_t i = tid; i < ny; i += kThreads) yo[i] = b8;
  }
}

// max(m, |a|, |b|) as one v_max3_f32 with absolute-value source modifiers.
// (fmaxf on values the compiler cannot prove quiet costs a canonicalising
// max per element first.)  These maxima only set operand scales; no NaN
// reaches them from valid inputs.
__device__ __forceinline__ float amax3(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}
template <int kW>
__device__ __forceinline__ float max_abs(float m, const float (&x)[kW]) {
  static_assert(kW % 2 == 0, "pairs");
#pragma unroll
  for (int e = 0; e < kW; e += 2) m = amax3(m, x[e], x[e + 1]);
  return m;
}
__device__ __forceinline__ float max4(float m, f4v x) { return amax3(amax3(m, x[0], x[1]), x[2], x[3]); }

// The group's partial sums added in the fixed order of the workgroups
// (0 + 1 + ... + kG-1), identical in every workgroup: `own` is workgroup h's
// partial, pt[m] the partial of its m-th partner in increasing order
// (workgroup m for m < h, m + 1 above).  h is uniform, so one branch picks
// the instance whose positions are known at compile time.
template <int kG, int kW, int kHh = 0>
__device__ __forceinline__ void ordered_sum(int h, const float (&own)[kW], const float (&pt)[kG - 1][kW],
                                            float (&out)[kW]) {
  if constexpr (kG == 2) {
#pragma unroll
    for (int e = 0; e < kW; ++e) out[e] = h == 0 ? own[e] + pt[0][e] : pt[0][e] + own[e];
  } else if constexpr (kHh < kG) {
    if (h == kHh) {
#pragma unroll
      for (int e = 0; e < kW; ++e) {
        float acc = kHh == 0 ? own[e] : pt[0][e];
#pragma unroll
        for (int gg = 1; gg < kG; ++gg) acc += gg < kHh ? pt[gg][e] : gg == kHh ? own[e] : pt[gg - 1][e];
        out[e] = acc;
      }
      return;
    }
    ordered_sum<kG, kW, kHh + 1>(h, own, pt, out);
  }
}

// kRW: retrieval after each token's write (true) or at the chunk-start
// state (false: y_j = M_{W_0}(q_j), without the masked correction terms).
// NW: waves per workgroup (Grp<NW>).  kEarly: move each chunk's inputs into
// LDS during the previous chunk (eight waves only; see `early`).  kSplit:
// each half's retrieval on a workgroup of its own (few streams; see is_r).
template <bool kRW, int NW, bool kEarly, bool kSplit>
__global__ void __launch_bounds__(64 * NW, 1) mlp2_group_kernel(Params p) {
  using C = Grp<NW>;
  static_assert(!kSplit || (kRW && NW == 8 && !kEarly), "the split runs eight-wave read-after-write workgroups");
  constexpr int kWaves = C::kWaves, kThreads = C::kThreads, kUG = C::kUG, kG = C::kG, kT = C::kT, kE = C::kE;
  constexpr int kYPer = C::kYPer;
  constexpr int OFF_A1 = C::OFF_A1, OFF_H1 = C::OFF_H1, OFF_W2 = C::OFF_W2, OFF_S2 = C::OFF_S2,
                OFF_COEF = C::OFF_COEF, OFF_STAGE = C::OFF_STAGE;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* sK = (_Float16*)(smem + OFF_K);
  _Float16* sQ = (_Float16*)(smem + OFF_Q);
  _Float16* sD2T = (_Float16*)(smem + OFF_D2T);
  _Float16* sSC = (_Float16*)(smem + OFF_SC);
  float* sDM = (float*)(smem + OFF_DM);
  _Float16* sA1 = (_Float16*)(smem + OFF_A1);
  _Float16* sH1 = (_Float16*)(smem + OFF_H1);
  _Float16* sW2 = (_Float16*)(smem + OFF_W2);
  _Float16* sS2 = (_Float16*)(smem + OFF_S2);
  float* cf = (float*)(smem + OFF_COEF);
  _Float16* ch = (_Float16*)(smem + OFF_COEF + COEF_H16);
  int* ci = (int*)(smem + OFF_COEF + COEF_INT);

  const int tid0 = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  // The thread index is re-read at the top of every chunk (see `relane`):
  // every LDS and global address of the chunk is derived from it, and the
  // compiler would otherwise hoist dozens of such addresses out of the chunk
  // loop and spill them.
  int tid = tid0, lane = tid0 & 63, lc = lane & 15, g = lane >> 4;
  // D[j][i] with the part carried over from row 31 (rows 32..63 of columns
  // 0..31; see the a1 stage); the condition is uniform in every caller's wave
  auto d_full = [&](int j, int i) {
    float d = sDM[j * RF + i];
    if (j >= 32 && i < 32)
      d = fmaf(cf[COEF_T11 + j - 32], sDM[31 * RF + i], fmaf(cf[COEF_T12 + j - 32], cf[COEF_XT + i], d));
    return d;
  };
  // D over the 16x16 tile of row block tr and column block tb: lane (g, lc)
  // gets rows 16 tr + 4g + r of column 16 tb + lc.  The part carried over
  // from row 31 (d_full) concerns only the tiles below row 32 and left of
  // column 32, a condition uniform over the wave.
  auto d_tile = [&](int tr, int tb) {
    const int col = 16 * tb + lc;
    f4v d;
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = sDM[(16 * tr + 4 * g + r) * RF + col];
    if (tr >= 2 && tb < 2) {
      const float d31 = sDM[31 * RF + col], xt = cf[COEF_XT + col];
      const f4v t11 = *(const f4v*)(cf + COEF_T11 + 16 * tr + 4 * g - 32);
      const f4v t12 = *(const f4v*)(cf + COEF_T12 + 16 * tr + 4 * g - 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = fmaf(t11[r], d31, fmaf(t12[r], xt, d[r]));
    }
    return d;
  };
  auto relane = [&] {
    int t = tid0;
    asm volatile("" : "+v"(t));
    tid = t;
    lane = t & 63;
    lc = lane & 15;   // row / column inside a 16x16 tile
    g = lane >> 4;    // K group; accumulator rows 4g .. 4g+3
  };

  // group / workgroup in it: blocks b, b + 8, b + 16, ... usually share an
  // XCD (round-robin dispatch), so groups are formed that way when the grid
  // allows it; correctness does not depend on the placement
  constexpr int kGS = kSplit ? 2 * kG : kG;   // workgroups per group
  int grp, h;
  {
    const int b = blockIdx.x;
    if (gridDim.x % (8 * kGS) == 0) {
      const int slot = b >> 3;
      grp = (b & 7) + 8 * (slot / kGS);
      h = slot % kGS;
    } else {
      grp = b / kGS;
      h = b % kGS;
    }
  }
  // With kSplit, workgroups kG .. 2 kG - 1 of a group are retrieval
  // workgroups: the one of half h (h = its index - kG) takes from the
  // key-side workgroup of that half, per chunk, the state copies, A1, Delta2,
  // Delta1 and the query products the read needs, and computes the chunk's
  // y (a5) one step behind, while the key side goes on with the next chunk.
  const bool is_r = kSplit && h >= kG;
  if (is_r) h -= kG;
  const int uw = kUW * w;               // this wave's first unit inside the workgroup's kUG
  const int hs = kUG * h + uw;          // ... and inside the layer's 256
  // the workgroup-level output tiles of this wave (O, y: tokens tj, columns
  // tc0 .. tc0 + kT - 1; the masked scores: tokens tj, keys tc0 ..)
  const int tj = (w * kT) >> 2, tc0 = (w * kT) & 3;
  // y rows kYRows h .. kYRows (h + 1) - 1 of a chunk are finished by
  // workgroup h: the waves whose tiles lie there park them in LDS, the
  // other workgroups' waves of those rows send theirs to it, and every
  // thread of it then sums kYPer elements (one row of 64 per wave and step)
  const int y_owner = (tj * kG) >> 2;
  const bool keeps_y = y_owner == h;
  // element of the owner's rows of this lane's tile element (i, r), and the
  // exchange word holding its rows r = 2 rp, 2 rp + 1: word k carries rows
  // 2 (k / 64), 2 (k / 64) + 1 of the owner's rows, column k % 64
  auto y_elem = [&](int i, int r) { return (16 * tj + 4 * g + r - C::kYRows * y_owner) * kD + 16 * (tc0 + i) + lc; };
  auto y_word = [&](int i, int rp) {
    return ((16 * tj + 4 * g - C::kYRows * y_owner) / 2 + rp) * kD + 16 * (tc0 + i) + lc;
  };
  // the wave that produced tiles (tt, 2 kk) and (tt, 2 kk + 1) of a masked
  // score matrix, whose scale the kk-th K-step of a product over keys uses
  auto score_wave = [](int tt, int kk) { return (4 * tt + 2 * kk) / kT; };

  unsigned long long* xw =
      (unsigned long long*)(p.xbuf + (int64_t)grp * (kSplit ? C::kGroupBytesSplit : C::kGroupBytes));
  // the hand-over words of this workgroup's half, parity par (word e of
  // thread t at e kThreads + t), and the receipts of its retrieval workgroup
  auto xP = [&](unsigned par) {
    return xw + C::kXOWords + C::kXYWords + ((int64_t)h * 2 + par) * C::kPubW * kThreads;
  };
  unsigned long long* const xA = xw + C::kXOWords + C::kXYWords + C::kXPWords + (int64_t)h * kThreads;
  // O partials of workgroup wg, parity par
  auto xO = [&](int wg, unsigned par) { return xw + ((int64_t)wg * 2 + par) * kThreads * (kE / 2); };
  // y partials sent by workgroup snd to its receiver slot sl
  // ((receiver - snd - 1) mod kG), parity par
  auto xY = [&](int snd, int sl, unsigned par) {
    return xw + C::kXOWords + (((int64_t)snd * (kG - 1) + sl) * 2 + par) * (C::kYElems / 2);
  };
  // the m-th partner in increasing order
  auto partner = [&](int m) { return m < h ? m : m + 1; };

  // a workgroup that gives up waiting for a partner records it (status
  // word, and the workgroup's flag checked at its next barrier)
  auto give_up = [&] {
    ci[INT_FAIL] = 1;
    __hip_atomic_store(p.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  bool failed = false;
  if (tid0 == 0) ci[INT_FAIL] = 0;

  // The y tiles of the previous chunk a keeping thread finishes (rows
  // 16 tj + 4g + r, columns 16 (tc0 + i) + lc) wait across the chunk
  // boundary in an LDS area of their own.  Registers would be spilled across
  // the boundary, and every reload from scratch would wait for the exchange
  // stores in flight.
  float* ypark = (float*)(smem + OFF_YP);   // kYElems floats: this workgroup's partial of its y rows
  int64_t prev_row0 = -1;   // global token row of the previous chunk's first token
  int prev_n = 0;
  unsigned seq = 0;         // sequence number of the current chunk (1, 2, ...)
  bool staged = false;      // the staging area holds the rows of the chunk about to start
                            // (eight waves: of the chunk after the current one)
  // With eight waves and early_inputs set, the chunk inputs are moved from
  // the staging area into their LDS tiles by waves 4..7 at the end of the
  // previous chunk, while waves 0..3 compute y (sK, sQ and the gate slots
  // are free by then): the chunk then starts without that stage and its
  // barrier.  (Measured: 2% faster with few streams; 0.5% slower with every
  // CU busy, where y's waves lose more to the sharing than the chunk start
  // gains.)
  constexpr bool early = kEarly && NW == 8;
  bool pre = false;         // the tiles already hold the inputs of the chunk about to start
  // the half-workgroup share of the staged chunk: pieces t and t + 256,
  // moved by the same threads that prefetched them (t = tid - 256 on waves
  // 4..7, t = tid on waves 0..3), into the K and Q tiles dK, dQ; returns
  // max |K| over the pieces, and the gates of token t (t < 64) in g3
  auto inputs_to_lds = [&](int nn, int t, _Float16* dK, _Float16* dQ, float3& g3) {
    const ChunkRegs<2> cr = unstage_chunk_regs<256>(smem + OFF_STAGE, nn, t);
    float kn = 0.f;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int piece = t + rr * 256, j = piece >> 3, cb = (piece & 7) * 8;
      const uint4 ku = cr.k[rr];
      const h8 kv = bf16x8_to_h8(ku), qv = bf16x8_to_h8(cr.q[rr]);
      kn = amax3(amax3(kn, bf16_lo(ku.x), bf16_hi(ku.x)), bf16_lo(ku.y), bf16_hi(ku.y));
      kn = amax3(amax3(kn, bf16_lo(ku.z), bf16_hi(ku.z)), bf16_lo(ku.w), bf16_hi(ku.w));
      *(h8*)(dK + j * RS + cb) = kv;
      *(h8*)(dQ + j * RS + cb) = qv;
    }
    g3 = make_float3(cr.ga, cr.ge, cr.gt);
    return kn;
  };
  auto gates_to_lds = [&](int t, float3 g3) {
    if (t < kB) {
      cf[COEF_THETA + t] = g3.z;
      float2* pairs = (float2*)(smem + OFF_COEF + COEF_PAIR);
      pairs[t] = make_float2(1.f - g3.x, g3.y);
    }
  };

  // the partners' partials of this thread's y elements for the chunk
  // numbered `tag`: words tid + kThreads e, i.e. rows 2 (w + kWaves e) and
  // 2 (w + kWaves e) + 1 of this workgroup's rows, column `lane`
  auto load_prev_y = [&](unsigned tag, float (&pv)[kG - 1][kYPer]) {
    const unsigned long long* bases[kG - 1];
#pragma unroll
    for (int m = 0; m < kG - 1; ++m) {
      const int snd = partner(m);
      bases[m] = xY(snd, (h - snd - 1 + kG) % kG, tag & 1u);
    }
    if (!tpoll<kThreads, kYPer / 2, kG - 1>(bases, tid, tag, p.spin_max, pv)) give_up();
  };
  // the fixed-order sum of the group's partials, stored as bf16 (value
  // 2e + q is row kYRows h + 2 (w + kWaves e) + q, column `lane`)
  auto finish_prev_y = [&](const float (&pv)[kG - 1][kYPer]) {
    float own[kYPer], sum[kYPer];
#pragma unroll
    for (int e = 0; e < kYPer; ++e) own[e] = ypark[(2 * (w + kWaves * (e >> 1)) + (e & 1)) * kD + lane];
    ordered_sum<kG, kYPer>(h, own, pv, sum);
#pragma unroll
    for (int e = 0; e < kYPer; ++e) {
      const int j = C::kYRows * h + 2 * (w + kWaves * (e >> 1)) + (e & 1);
      if (j < prev_n) p.y[(prev_row0 + j) * kD + lane] = __float2bfloat16(sum[e]);
    }
  };
  // ================= a1: coefficients (every workgroup computes them identically) =================
  // On the key side while the O exchange is in flight.  Lane m of a wave
  // holds token m's (1 - alpha_m, eta_m); padding tokens have alpha = 0,
  // eta = 1, theta = 0.
  //
  // D, one lane per column i: t = theta_i prod_{i<m<=j} eta_m, started at
  // j == i by adding theta_i to a zero product, and
  // D[j][i] = (1 - alpha_j) D[j-1][i] + t -- one fma per row on each of the
  // two carried values, the row's gates broadcast from LDS.  Wave kWD0
  // runs rows 0..31 and wave kWD1 rows 32..63, each starting from zero.
  // For columns i >= 32 the second wave's rows are exact (their
  // recurrences start at row i); for i < 32 they lack the part carried
  // over from row 31,
  // which every reader adds (d_full) through the column-independent
  // transfer
  //   (D, t)_j += (T11_j D_31 + T12_j t_31, T22_j t_31),
  // T11_j = prod_{32<=m<=j} (1 - alpha_m), T22_j = prod_{32<=m<=j} eta_m,
  // T12_j = sum_{32<=l<=j} prod_{l<m<=j} (1 - alpha_m) T22_l,
  // which wave kWS gets from prefix scans restarted at row 32, beside E_j (a
  // prefix product of eta) and (A_j, F_j) (a prefix scan of the maps
  // u -> (1 - alpha_j) u + E_j: A_j is the scan's product part, F_j its
  // value from F_{-1} = 0).  First read after the next barrier.
  auto coef_stage = [&](auto&& mid) {
    if (w == C::kWD0 || w == C::kWD1) {
      const int i = lane;
      const int j0 = w == C::kWD0 ? 0 : 32;
      const float thi = cf[COEF_THETA + i];
      float di = 0.f, t = 0.f;
      const float4* pairs4 = (const float4*)(smem + OFF_COEF + COEF_PAIR) + j0 / 2;
#pragma unroll 2
      for (int b = 0; b < 4; ++b) {
        // halfway through the recurrence (the key side's first poll of
        // the partner's O goes out here; its tags are checked after the stage)
        if (b == 2) mid();
        // 8 rows per batch: the steps' (1 - alpha_j, eta_j) pairs as LDS
        // broadcasts (two steps per 16-byte read), the rows stored after
        // the batch so that the gate reads never wait behind row stores
        float4 gq[4];
        float drows[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) gq[q] = pairs4[4 * b + q];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + 8 * b + jj;
          const float ga = (jj & 1) ? gq[jj >> 1].z : gq[jj >> 1].x;
          const float ge = (jj & 1) ? gq[jj >> 1].w : gq[jj >> 1].y;
          const float inj = i == j ? thi : 0.f;   // theta_i enters at row i
          t = fmaf(ge, t, inj);
          di = fmaf(ga, di, t);
          drows[jj] = di;
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sDM[(j0 + 8 * b + jj) * RF + i] = drows[jj];
      }
      // wave kWD0: t at row 31 for i < 32; wave kWD1: t at row 63 (= U_i) for i >= 32
      if ((w == C::kWD0) == (i < 32)) cf[COEF_XT + i] = t;
    } else if (w == C::kWS) {
      const float2 gl = ((const float2*)(smem + OFF_COEF + COEF_PAIR))[lane];
      const float e = wave_prefix_prod(gl.y);
      float a = gl.x, f = e;
      wave_affine_scan(a, f);
      cf[COEF_A + lane] = a;
      cf[COEF_E + lane] = e;
      cf[COEF_F + lane] = f;
      // the same scans restarted at row 32 (identity maps below it)
      const bool lo = lane < 32;
      const float eb = wave_prefix_prod(lo ? 1.f : gl.y);
      float a2 = lo ? 1.f : gl.x, f2b = lo ? 0.f : eb;
      wave_affine_scan(a2, f2b);
      if (!lo) {
        cf[COEF_T11 + lane - 32] = a2;
        cf[COEF_T12 + lane - 32] = f2b;
      }
      if (lane == 63) ci[INT_T22] = __float_as_int(eb);
    }
  };
  // the fold weights of token i: U_i and D[n-1][i], each scaled into
  // (0.5, 1] for fp16 (one wave, lane per token)
  auto store_fold_weights = [&](int i, float ui, float dlast) {
    const float mu = wave_max(fabsf(ui)), md = wave_max(fabsf(dlast));
    int eu = 0, ed = 0;
    if (mu > 0.f && mu < INFINITY) { (void)frexpf(mu, &eu); eu = -eu; }
    if (md > 0.f && md < INFINITY) { (void)frexpf(md, &ed); ed = -ed; }
    ch[H16_WU + i] = (_Float16)ldexpf(ui, eu);
    ch[H16_WD + i] = (_Float16)ldexpf(dlast, ed);
    if (lane == 0) { ci[INT_EWU] = eu; ci[INT_EWD] = ed; }
  };
  // The key side of a split launch needs no D matrix (only the reads do):
  // wave kWS scans A, E, F as above, and wave kWD0 gets the fold weights from
  // scans over the lanes in reversed token order (lane l holds token
  // i = 63 - l):
  //   U_i = theta_i prod_{i<m} eta_m,
  //   D[n-1][i] = theta_i R_i,  R_i = a_i + eta_{i+1} R_{i+1},  R_64 = 0,
  //   a_i = prod_{i<m<=n-1} (1 - alpha_m) for i <= n-1, 0 beyond,
  // which is D's recurrence summed along its last row (padding tokens carry
  // alpha = 0, eta = 1, so the products may run to token 63).
  auto key_coef_stage = [&](int n) {
    const float2* pairs = (const float2*)(smem + OFF_COEF + COEF_PAIR);
    if (w == C::kWS) {
      const float2 gl = pairs[lane];
      const float e = wave_prefix_prod(gl.y);
      float a = gl.x, f = e;
      wave_affine_scan(a, f);
      cf[COEF_A + lane] = a;
      cf[COEF_E + lane] = e;
      cf[COEF_F + lane] = f;
    } else if (w == C::kWD0) {
      const int i = 63 - lane;
      float2 gn = make_float2(1.f, 1.f);   // token i + 1's (1 - alpha, eta); none after token 63
      if (lane > 0) gn = pairs[i + 1];
      const float pa = wave_prefix_prod(gn.x), pe = wave_prefix_prod(gn.y);
      float c = gn.y, r = i <= n - 1 ? pa : 0.f;
      wave_affine_scan(c, r);
      const float th = cf[COEF_THETA + i];
      store_fold_weights(i, th * pe, th * r);
    }
  };

  // the raw first-layer scores Q K^T, tiles (tj, tc0 + i)
  auto raw_scores = [&](f4v (&scr)[kT]) {
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      f4v acc = {};
      const _Float16* arow = sQ + (16 * tj + lc) * RS;
      const _Float16* brow = sK + (16 * (tc0 + i) + lc) * RS;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc = mfma(frag_c8(arow, 32 * kk, g), frag_c8(brow, 32 * kk, g), acc);
      scr[i] = acc;
    }
  };
  // first-layer masked scores SC1 = D o (Q K^T) into sSC [key][query], tiles
  // (tj, tc0 + i), with this wave's own scale
  auto sc1_store = [&](const f4v (&scr)[kT]) {
    float sc[kE], am = 0.f;
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const f4v dt = d_tile(tj, tc0 + i);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[4 * i + r] = scr[i][r] * dt[r];
    }
    am = wave_max(max_abs(am, sc));
    const int esc = scale_exp(am);
    const float fsc = pow2pos(esc);
#pragma unroll
    for (int i = 0; i < kT; ++i)
      store_rows4(sSC, RS, 16 * (tc0 + i) + lc, 16 * tj + 4 * g,
                  h4{sc16(sc[4 * i], fsc), sc16(sc[4 * i + 1], fsc), sc16(sc[4 * i + 2], fsc),
                     sc16(sc[4 * i + 3], fsc)});
    if (lane == 0) ci[INT_ESC + w] = esc;
  };
  // ================= a5 layer 1: Zq1 = diag(A) Q W1^T + diag(F) Q S1^T - SC1 Delta1 =================
  // H1 = SiLU(Zq1) over this wave's units (rows: query tiles), in units of
  // -1/ln 2; main(tt) gives the first two terms of query tile tt in those units
  auto zq1_h1 = [&](auto&& main, const h8 (&d1f)[2], int eD1, f4v (&H1f)[4]) {
    float am = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f4v z = main(tt);
      if constexpr (kRW) {
        // the masked term's two K-steps carry the scales of the waves that produced them
        f4v m0 = {}, m1v = {};
        m0 = mfma(frag_tr_rk(sSC, RS, 0, 16 * tt, g, lc), d1f[0], m0);
        m1v = mfma(frag_tr_rk(sSC, RS, 32, 16 * tt, g, lc), d1f[1], m1v);
        const float c30 = pow2neg(eD1 + ci[INT_ESC + score_wave(tt, 0)]) * kLog2e,
                    c31 = pow2neg(eD1 + ci[INT_ESC + score_wave(tt, 1)]) * kLog2e;
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = fmaf(m0[r], c30, fmaf(m1v[r], c31, z[r]));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) H1f[tt][r] = z[r] * sigmoid_x(z[r]);   // -H1 log2 e
      am = max4(am, H1f[tt]);
    }
    const float wam = wave_max(am);
    if (lane == 0) ci[INT_MH1 + w] = __float_as_int(wam);
  };
  // H1 with the workgroup-wide scale (its exponent returned), copied [u][j]
  // for the scores and y; after a barrier that follows every wave's zq1_h1
  auto h1_copy = [&](const f4v (&H1f)[4]) {
    float mm = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) mm = fmaxf(mm, __int_as_float(ci[INT_MH1 + i]));
    const int eH1 = scale_exp(mm * kLn2);   // the waves' maxima are of |H1| log2 e
    const float fH = pow2pos(eH1) * -kLn2;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) store_rows4(sH1, RS, uw + lc, 16 * tt + 4 * g, to_h4(H1f[tt], fH));
    return eH1;
  };
  // ================= masked second-layer scores D o (H1 A1^T): tiles (tj, tc0 + i) =================
  // into sSC [key][query], with this wave's own scale
  auto p_scores = [&](int eH1, int eA1) {
    float pv[kE], am = 0.f;
    const float cp = pow2neg(eH1 + eA1);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      f4v acc = {};
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk)
        acc = mfma(frag_tr_c8(sH1, RS, 32 * kk, 16 * tj, g, lc), frag_tr_c8(sA1, RS, 32 * kk, 16 * (tc0 + i), g, lc),
                   acc);
      const f4v dt = d_tile(tj, tc0 + i);
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[4 * i + r] = acc[r] * cp * dt[r];
    }
    am = wave_max(max_abs(am, pv));
    const int edp = scale_exp(am);
    const float fdp = pow2pos(edp);
#pragma unroll
    for (int i = 0; i < kT; ++i)
      store_rows4(sSC, RS, 16 * (tc0 + i) + lc, 16 * tj + 4 * g,
                  h4{sc16(pv[4 * i], fdp), sc16(pv[4 * i + 1], fdp), sc16(pv[4 * i + 2], fdp),
                     sc16(pv[4 * i + 3], fdp)});
    if (lane == 0) ci[INT_EDP + w] = edp;
  };
  // ================= a5 layer 2: y = diag(A) H1 W2^T + diag(F) H1 S2^T - (D o P) Delta2 =================
  // after a barrier that follows every wave's H1 copy and scores; the rows of
  // other workgroups are sent to them (tagged `seq`, parity `par`)
  auto y_stage = [&](int eH1, int e2, int eD2, unsigned par) {
    if constexpr (NW == 8) {
      // Four 32 x 32 blocks on v_mfma_f32_32x32x16_f16, one per wave of
      // waves 0..3 (one per SIMD): block (jb, cb) = (32 (w >> 1), 32 (w & 1)).
      // Each operand block is read from LDS once per block, against twice
      // (H1, P) or four times (W2^T, S2^T, Delta2^T) over the eight waves'
      // 16 x 16 tile pairs; the stage is bound by these reads.
      if (w < 4) {
        const int jb = 32 * (w >> 1), cb = 32 * (w & 1);
        const int l32 = lane & 31, hk = lane >> 5, grp16 = lane >> 4;
        // fragment of block columns n0 .. n0 + 31 over K rows kb .. kb + 15 of a K-major tile
        auto fr32 = [&](const _Float16* T, int kb, int n0) {
          const int k0 = kb + 8 * (grp16 >> 1), nn = n0 + 16 * (grp16 & 1);
          const h4 lo = tr4(T, RS, k0, nn, lc), hi = tr4(T, RS, k0 + 4, nn, lc);
          return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        f16v aw = {}, as = {};
#pragma unroll
        for (int ks = 0; ks < kUG / 16; ++ks) {
          const h8 hf = fr32(sH1, 16 * ks, jb);
          aw = mfma32(hf, fr32(sW2, 16 * ks, cb), aw);
          if constexpr (kRW) as = mfma32(hf, fr32(sS2, 16 * ks, cb), as);
        }
        if constexpr (kRW) {
          // operand reads two K-steps ahead of the products (the reads'
          // latency, not the matrix unit, bounds the chain otherwise)
          __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
          for (int ks = 0; ks < kUG / 16; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (ks + 2 < kUG / 16) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
          }
        }
        float yv[16];
        const float cy = pow2neg(eH1 + e2);
        if constexpr (kRW) {
          // the masked term over keys 0..31 and 32..63 separately: each half
          // of a query tile's scores carries the scale of the wave that produced it
          f16v m0 = {}, m1v = {};
          const _Float16* drow = sD2T + (cb + l32) * RS + 8 * hk;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) m0 = mfma32(fr32(sSC, 16 * ks, jb), *(const h8*)(drow + 16 * ks), m0);
#pragma unroll
          for (int ks = 2; ks < 4; ++ks) m1v = mfma32(fr32(sSC, 16 * ks, jb), *(const h8*)(drow + 16 * ks), m1v);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int tjq = (jb >> 4) + (q >> 1);   // the query tile of rows jb + 8q + 4hk ..
            const float c30 = pow2neg(eD2 + ci[INT_EDP + score_wave(tjq, 0)]),
                        c31 = pow2neg(eD2 + ci[INT_EDP + score_wave(tjq, 1)]);
            const f4v av = *(const f4v*)(cf + COEF_A + jb + 8 * q + 4 * hk);
            const f4v fv = *(const f4v*)(cf + COEF_F + jb + 8 * q + 4 * hk);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int r = 4 * q + rr;
              const float main = fmaf(av[rr], aw[r], fv[rr] * as[r]) * cy;
              yv[r] = fmaf(m0[r], -c30, fmaf(m1v[r], -c31, main));
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) yv[r] = aw[r] * cy;
        }
        // keep the block if its rows are this workgroup's, else send them
        // (element / word indexing of the owner's rows as in finish_prev_y)
        const int owner = jb / C::kYRows;
        if (owner == h) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ypark[(jb + 8 * (r >> 2) + 4 * hk + (r & 3) - C::kYRows * h) * kD + cb + l32] = yv[r];
        } else {
          unsigned long long* yb = xY(h, (owner - h - 1 + kG) % kG, par);
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            tstore(yb, ((jb + 8 * (r >> 2) + 4 * hk + (r & 3) - C::kYRows * owner) / 2) * kD + cb + l32, yv[r],
                   yv[r + 1], seq);
        }
      }
    } else {
      float yv[kE];
      const float cy = pow2neg(eH1 + e2);
      const f4v av = *(const f4v*)(cf + COEF_A + 16 * tj + 4 * g);
      const f4v fv = *(const f4v*)(cf + COEF_F + 16 * tj + 4 * g);
#pragma unroll
      for (int i = 0; i < kT; ++i) {
        const int crow = 16 * (tc0 + i) + lc;
        f4v aw = {}, as = {};
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
          const h8 hf = frag_tr_c8(sH1, RS, 32 * kk, 16 * tj, g, lc);
          aw = mfma(hf, frag_tr_c8(sW2, RS, 32 * kk, 16 * (tc0 + i), g, lc), aw);
          if constexpr (kRW) as = mfma(hf, frag_tr_c8(sS2, RS, 32 * kk, 16 * (tc0 + i), g, lc), as);
        }
        if constexpr (kRW) {
          f4v m0 = {}, m1v = {};
          m0 = mfma(frag_tr_c8(sSC, RS, 0, 16 * tj, g, lc), frag_c8(sD2T + crow * RS, 0, g), m0);
          m1v = mfma(frag_tr_c8(sSC, RS, 32, 16 * tj, g, lc), frag_c8(sD2T + crow * RS, 32, g), m1v);
          const float c30 = pow2neg(eD2 + ci[INT_EDP + score_wave(tj, 0)]),
                      c31 = pow2neg(eD2 + ci[INT_EDP + score_wave(tj, 1)]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float main = fmaf(av[r], aw[r], fv[r] * as[r]) * cy;
            yv[4 * i + r] = fmaf(m0[r], -c30, fmaf(m1v[r], -c31, main));
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) yv[4 * i + r] = aw[r] * cy;
        }
      }
      // keep my rows, send the other rows to the workgroup that finishes them
      if (keeps_y) {
#pragma unroll
        for (int i = 0; i < kT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) ypark[y_elem(i, r)] = yv[4 * i + r];
      } else {
        unsigned long long* yb = xY(h, (y_owner - h - 1 + kG) % kG, par);
#pragma unroll
        for (int i = 0; i < kT; ++i)
#pragma unroll
          for (int rp = 0; rp < 2; ++rp) tstore(yb, y_word(i, rp), yv[4 * i + 2 * rp], yv[4 * i + 2 * rp + 1], seq);
      }
    }
  };
  __syncthreads();

  // ================= the retrieval workgroup of half h (kSplit) =================
  // Per chunk: the inputs, the coefficients and the first-layer masked
  // scores of its own; the key side's words of the chunk (partly requested
  // before that work, so that a workgroup behind the key side finds them
  // arrived), then a5 exactly as the unsplit kernel runs it.  The receipt,
  // sent at the end of the chunk, lets the key side reuse the words' slot
  // two chunks later; the y rows cross between the retrieval pair as in the
  // unsplit kernel, one chunk late.  The partner's y of chunk seq - 1 is read
  // before this chunk's y is sent, so a slot is rewritten only after it was
  // read.
  if constexpr (kSplit) {
    if (is_r) {
      for (int s = grp; s < p.streams && !failed; s += p.n_groups) {
        const int64_t tok0 = (int64_t)s * p.N;
        for (int c0 = 0, cidx = 0; c0 < p.N; c0 += p.chunk, ++cidx) {
          const int n = min(p.chunk, p.N - c0);
          relane();
          ++seq;
          const int stamp_slot = (TM_STAGE_STAMPS && TM_STAMP_R && grp == 0 && h == 0 && s == grp &&
                                  cidx >= kStampFrom && cidx < kStampFrom + kStampChunks) ? cidx - kStampFrom : -1;
          (void)stamp_slot;
          STAMP(0);
          const unsigned par = seq & 1u;
          int next_s = s, next_c0 = c0 + p.chunk, next_ci = cidx + 1;
          if (next_c0 >= p.N) { next_s = s + p.n_groups; next_c0 = 0; next_ci = 0; }
          const bool has_next = next_s < p.streams && p.N > 0;
          if (tid == 0) ci[INT_FAIL] = 0;
          // the chunk's K, Q (fp16) and gates into LDS, unless waves 4..7
          // moved them in during the previous chunk's y
          if (!pre) {
            const ChunkRegs<C::kRowPasses> cr =
                staged ? unstage_chunk_regs<kThreads>(smem + OFF_STAGE, n, tid)
                       : load_chunk_regs<kThreads>(p, tok0 + c0, gate_base(p, s, cidx, c0), n, tid);
#pragma unroll
            for (int rr = 0; rr < C::kRowPasses; ++rr) {
              const int piece = tid + rr * kThreads, j = piece >> 3, cb = (piece & 7) * 8;
              *(h8*)(sK + j * RS + cb) = bf16x8_to_h8(cr.k[rr]);
              *(h8*)(sQ + j * RS + cb) = bf16x8_to_h8(cr.q[rr]);
            }
            if (tid < kB) {
              cf[COEF_THETA + tid] = cr.gt;
              float2* pairs = (float2*)(smem + OFF_COEF + COEF_PAIR);
              pairs[tid] = make_float2(1.f - cr.ga, cr.ge);
            }
            STAMP(1);
            __syncthreads();   // the chunk's tiles and gates
            // the next chunk's rows to the staging area, by the waves that
            // move them into the tiles during this chunk's y (waited for at
            // once, as during y: only a workgroup's first chunk comes here)
            if (has_next && w >= 4) {
              prefetch_chunk_lds<256>(p, (int64_t)next_s * p.N + next_c0, gate_base(p, next_s, next_ci, next_c0),
                                      min(p.chunk, p.N - next_c0), tid - 256, smem + OFF_STAGE);
              __builtin_amdgcn_s_waitcnt(0x0F70);
            }
            staged = has_next;
          } else {
            STAMP(1);
          }
          // The key side's words of this chunk: the copies' words loaded
          // across the coefficient stage by the waves that have no
          // recurrence there (all 44 in flight would spill registers), the
          // rest after the coefficients' barrier, with the partner's y of
          // the previous chunk (by then its stores have landed).
          const unsigned long long* pb = xP(par);
          TagWords<kThreads, C::kPubW> pw;
          const unsigned long long* ybases[kG - 1];
#pragma unroll
          for (int m = 0; m < kG - 1; ++m) {
            const int snd = partner(m);
            ybases[m] = xY(snd, (h - snd - 1 + kG) % kG, (seq - 1) & 1u);
          }
          TPollEarly<kThreads, kYPer / 2, kG - 1> ypoll;
          const bool coef_wave = w == C::kWD0 || w == C::kWD1 || w == C::kWS;
          if (!coef_wave) pw.template issue<C::PW_1, C::PW_2>(pb, tid);
          STAMP(2);
          coef_stage([] {});
          STAMP(3);
          f4v scr[kT];
          raw_scores(scr);
          STAMP(4);
          __syncthreads();   // the coefficients
          STAMP(5);
          if (coef_wave) pw.template issue<C::PW_1, C::PW_2>(pb, tid);
          pw.template issue<C::PW_2, C::kPubW>(pb, tid);
          if (prev_row0 >= 0) ypoll.issue(ybases, tid);
          sc1_store(scr);
          STAMP(6);
          // the key side's words, in the order it writes them
          bool got = pw.template wait<C::PW_1, C::PW_2>(pb, tid, seq, p.spin_max);
          STAMP(7);
          got = got && pw.template wait<C::PW_2, C::PW_3>(pb, tid, seq, p.spin_max);
          STAMP(8);
          got = got && pw.template wait<C::PW_3, C::kPubW>(pb, tid, seq, p.spin_max);
          if (!got) give_up();
          STAMP(9);
          // the chunk-start W2^T, S2^T copies, A1^T and Delta2^T into their
          // tiles, where the key side keeps them (value e of a group: word
          // e / 3 of the group, place e % 3)
          auto hval = [&](int w0, int e) { return h3_get(pw.wd[w0 + e / 3], e % 3); };
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int b = 4 * ct;
            store_rows4(sW2, RS, uw + lc, 16 * ct + 4 * g,
                        h4{hval(C::PW_1, b), hval(C::PW_1, b + 1), hval(C::PW_1, b + 2), hval(C::PW_1, b + 3)});
            store_rows4(sS2, RS, uw + lc, 16 * ct + 4 * g,
                        h4{hval(C::PW_1, 16 + b), hval(C::PW_1, 17 + b), hval(C::PW_1, 18 + b), hval(C::PW_1, 19 + b)});
            store_rows4(sA1, RS, uw + lc, 16 * ct + 4 * g,
                        h4{hval(C::PW_1, 32 + b), hval(C::PW_1, 33 + b), hval(C::PW_1, 34 + b), hval(C::PW_1, 35 + b)});
          }
#pragma unroll
          for (int i = 0; i < kT; ++i)
            *(h4*)(sD2T + (16 * (tc0 + i) + lc) * RS + 16 * tj + 4 * g) =
                h4{hval(C::PW_2, 4 * i), hval(C::PW_2, 4 * i + 1), hval(C::PW_2, 4 * i + 2), hval(C::PW_2, 4 * i + 3)};
          const int e2 = h3_int(pw.wd[C::PW_1 + 16], 0), eA1 = h3_int(pw.wd[C::PW_1 + 16], 1),
                    eD2 = h3_int(pw.wd[C::PW_2 + 2], 2), eD1 = h3_int(pw.wd[C::PW_3 + 5], 1);
          // the query products: twords 3 .. 10 of the second group
          f4v mz[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const unsigned long long wd = pw.wd[C::PW_2 + 3 + 2 * tt + (r >> 1)];
              mz[tt][r] = (r & 1) ? tword_hi(wd) : tword_lo(wd);
            }
          h8 d1f[2];
#pragma unroll
          for (int e = 0; e < 16; ++e) d1f[e >> 3][e & 7] = hval(C::PW_3, e);
          // the previous chunk's y rows of this workgroup
          if (prev_row0 >= 0) {
            float pyv[kG - 1][kYPer];
            if (!ypoll.check(seq - 1, pyv) &&
                !tpoll<kThreads, kYPer / 2, kG - 1>(ybases, tid, seq - 1, p.spin_max, pyv))
              give_up();
            finish_prev_y(pyv);
          }
          STAMP(10);
          __syncthreads();   // every wave's first-layer scores and copies
          if (ci[INT_FAIL]) { failed = true; break; }
          STAMP(11);
          f4v H1f[4];
          zq1_h1([&](int tt) { return mz[tt]; }, d1f, eD1, H1f);
          STAMP(12);
          __syncthreads();   // every wave's H1 maximum
          STAMP(13);
          const int eH1 = h1_copy(H1f);
          STAMP(14);
          __syncthreads();   // every wave's H1 copy
          STAMP(15);
          p_scores(eH1, eA1);
          STAMP(16);
          __syncthreads();   // every wave's second-layer scores
          STAMP(17);
          y_stage(eH1, e2, eD2, par);
          // the next chunk's inputs into their tiles (waves 4..7, beside y
          // on waves 0..3; K and Q are not read after the raw scores), then
          // the chunk after it into the staging area
          if (staged && w >= 4) {
            // (this thread's staging loads have landed)
            __builtin_amdgcn_s_waitcnt(0x0F70);
            float3 g3;
            (void)inputs_to_lds(min(p.chunk, p.N - next_c0), tid - 256, sK, sQ, g3);
            gates_to_lds(tid - 256, g3);
            int s2 = next_s, c2 = next_c0 + p.chunk, i2 = next_ci + 1;
            if (c2 >= p.N) { s2 = next_s + p.n_groups; c2 = 0; i2 = 0; }
            if (s2 < p.streams) {
              // this thread's staging reads are complete before the slots it
              // read are refilled (the same threads refill them)
              __builtin_amdgcn_s_waitcnt(0xC07F);
              prefetch_chunk_lds<256>(p, (int64_t)s2 * p.N + c2, gate_base(p, s2, i2, c2), min(p.chunk, p.N - c2),
                                      tid - 256, smem + OFF_STAGE);
              // landed before the chunk ends (these waves wait for y anyway):
              // an LDS load still in flight across the loop would make the
              // next chunk's first barrier wait for every memory operation,
              // the key side's words requested before it included
              __builtin_amdgcn_s_waitcnt(0x0F70);
            }
          }
          // The receipt for this chunk's words (read long ago; sent last, as
          // any later wait for a load would also wait for this store)
          if (got) __hip_atomic_store(xA + tid, tword(0.f, 0.f, seq), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          pre = staged;
          if (staged) {
            int s2 = next_s, c2 = next_c0 + p.chunk;
            if (c2 >= p.N) { s2 = next_s + p.n_groups; c2 = 0; }
            staged = s2 < p.streams;
          }
          prev_row0 = tok0 + c0;
          prev_n = n;
          STAMP(18);
          __syncthreads();   // LDS tiles are rewritten by the next chunk
          STAMP(19);
          STAMP(20);
          STAMP(21);
          STAMP(22);
          STAMP(23);
        }
      }
      // the last chunk's y rows
      if (!failed && prev_row0 >= 0) {
        float pyv[kG - 1][kYPer];
        load_prev_y(seq, pyv);
        finish_prev_y(pyv);
        __syncthreads();
        if (ci[INT_FAIL]) failed = true;
      }
      if (failed) poison_group_streams<kThreads>(p, grp, tid);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      return;
    }
  }

  for (int s = grp; s < p.streams && !failed; s += p.n_groups) {
    const int64_t tok0 = (int64_t)s * p.N;
    // ---- this wave's state, VGPR-resident ----
    // W1s[ct]: rows c = 16 ct + 4g + r, lanes u = hs + lc   (W1[u][c])
    // W2s[ct]: rows c = 16 ct + 4g + r, lanes u = hs + lc   (W2[c][u])
    f4v W1s[4], S1s[4], W2s[4], S2s[4];
    {
      float m1 = 0.f, m2 = 0.f;   // this lane's max |S1| and max |W2|,|S2| (for the operand scales)
      float n1 = 0.f;             // this lane's max |W1| (a bound on the A1 scale; with m1, the layer-1 scale)
      const float* Wi = p.W_in + (int64_t)s * kP;
      const float* Si = p.S_in + (int64_t)s * kP;
      const int u = hs + lc;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = 16 * ct + 4 * g;
        W1s[ct] = *(const f4v*)(Wi + u * kD + c);
        S1s[ct] = *(const f4v*)(Si + u * kD + c);
        n1 = max4(n1, W1s[ct]);
        m1 = max4(m1, S1s[ct]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          W2s[ct][r] = Wi[kH * kD + (c + r) * kH + u];
          S2s[ct][r] = Si[kH * kD + (c + r) * kH + u];
        }
        m2 = max4(max4(m2, W2s[ct]), S2s[ct]);
      }
      const float wn1 = wave_max(n1), wm1 = fmaxf(wave_max(m1), wn1), wm2 = wave_max(m2);
      if (lane == 0) {
        ci[INT_M1 + w] = __float_as_int(wm1);
        ci[INT_M2 + w] = __float_as_int(wm2);
        ci[INT_N1 + w] = __float_as_int(wn1);
      }
    }
    // every wave's maxima before the first chunk reads them (a chunk whose
    // inputs were moved in early has no barrier before its key-side stage)
    if constexpr (early || kSplit) __syncthreads();

    for (int c0 = 0, cidx = 0; c0 < p.N; c0 += p.chunk, ++cidx) {
      const int n = min(p.chunk, p.N - c0);
      relane();
      ++seq;
      const int stamp_slot = (TM_STAGE_STAMPS && !TM_STAMP_R && grp == 0 && h == 0 && s == grp &&
                              cidx >= kStampFrom && cidx < kStampFrom + kStampChunks) ? cidx - kStampFrom : -1;
      (void)stamp_slot;
      STAMP(0);
      // (split) the receipt for this thread's hand-over words, checked
      // before the words of two chunks back are overwritten
      unsigned long long ackw = 0;
      if constexpr (kSplit) ackw = __hip_atomic_load(xA + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

      // the next chunk (in this stream or the group's next one)
      int next_s = s, next_c0 = c0 + p.chunk, next_ci = cidx + 1;
      if (next_c0 >= p.N) { next_s = s + p.n_groups; next_c0 = 0; next_ci = 0; }
      const bool has_next = next_s < p.streams && p.N > 0;
      if constexpr (early || kSplit) {
        if (tid == 0) {
          ci[INT_AMAX_D2] = 0;
          ci[INT_FAIL] = 0;
        }
      }
      // The key side of a split launch keeps two sets of K and Q tiles (the
      // y park and score areas, which only a retrieval workgroup uses, are
      // the second): waves 0..3 move the next chunk's inputs into the other
      // set after the O exchange, so a chunk starts without its input stage.
      if constexpr (kSplit) {
        const bool alt = seq & 1u;
        sK = (_Float16*)(smem + (alt ? OFF_YP : OFF_K));
        sQ = (_Float16*)(smem + (alt ? OFF_SC : OFF_Q));
      }

      // ================= the chunk's K, Q (fp16) and gates into LDS =================
      if (!((early || kSplit) && pre)) {
        // (this thread's staging loads were waited for after the previous
        // chunk's exchange; waiting here would also wait for the y exchange
        // stores just issued)
        const ChunkRegs<C::kRowPasses> cr =
            staged ? unstage_chunk_regs<kThreads>(smem + OFF_STAGE, n, tid)
                   : load_chunk_regs<kThreads>(p, tok0 + c0, gate_base(p, s, cidx, c0), n, tid);
        float kn = 0.f;
#pragma unroll
        for (int rr = 0; rr < C::kRowPasses; ++rr) {
          const int piece = tid + rr * kThreads, j = piece >> 3, cb = (piece & 7) * 8;
          const uint4 ku = cr.k[rr];
          const h8 kv = bf16x8_to_h8(ku), qv = bf16x8_to_h8(cr.q[rr]);
          // max |K| from the bf16 values: their fp16 conversion is exact in
          // fp16's normal range, and the A1 bound leaves a factor 4 of headroom
          kn = amax3(amax3(kn, bf16_lo(ku.x), bf16_hi(ku.x)), bf16_lo(ku.y), bf16_hi(ku.y));
          kn = amax3(amax3(kn, bf16_lo(ku.z), bf16_hi(ku.z)), bf16_lo(ku.w), bf16_hi(ku.w));
          *(h8*)(sK + j * RS + cb) = kv;
          *(h8*)(sQ + j * RS + cb) = qv;
        }
        if (tid < kB) {
          cf[COEF_THETA + tid] = cr.gt;
          float2* pairs = (float2*)(smem + OFF_COEF + COEF_PAIR);
          pairs[tid] = make_float2(1.f - cr.ga, cr.ge);
        }
        if constexpr (!early && !kSplit) {
          if (tid == 0) {
            ci[INT_AMAX_D2] = 0;
            ci[INT_FAIL] = 0;
          }
        }
        const float wnk = wave_max(kn);
        if (lane == 0) ci[INT_NK + w] = __float_as_int(wnk);
        STAMP(1);
        __syncthreads();
        // the next chunk's rows go straight to the staging area (with eight
        // waves by waves 4..7, which move them into the tiles at the end of
        // this chunk)
        if (has_next) {
          const int64_t r0 = (int64_t)next_s * p.N + next_c0, g0 = gate_base(p, next_s, next_ci, next_c0);
          const int nn = min(p.chunk, p.N - next_c0);
          if constexpr (early) {
            if (w >= 4) prefetch_chunk_lds<256>(p, r0, g0, nn, tid - 256, smem + OFF_STAGE);
          } else if constexpr (kSplit) {
            if (w < 4) prefetch_chunk_lds<256>(p, r0, g0, nn, tid, smem + OFF_STAGE);
          } else {
            prefetch_chunk_lds<kThreads>(p, r0, g0, nn, tid, smem + OFF_STAGE);
          }
        }
        staged = has_next;
      } else {
        STAMP(1);
        if constexpr (kSplit) {
          // the next chunk's rows to the staging area, by the threads that
          // moved this chunk's out of it (their reads of it complete first)
          if (has_next && w < 4) {
            __builtin_amdgcn_s_waitcnt(0xC07F);
            prefetch_chunk_lds<256>(p, (int64_t)next_s * p.N + next_c0, gate_base(p, next_s, next_ci, next_c0),
                                    min(p.chunk, p.N - next_c0), tid, smem + OFF_STAGE);
          }
          staged = has_next;
        }
      }
      STAMP(2);

      STAMP(3);
      // state scales: W1/S1 per wave; W2/S2 joint over the workgroup (the
      // workgroup's O and y partials are contractions over all its waves'
      // W2 and S2 copies)
      int e2;
      {
        float mm = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) mm = fmaxf(mm, __int_as_float(ci[INT_M2 + i]));
        e2 = scale_exp(mm);
      }
      const int e1 = scale_exp(__int_as_float(ci[INT_M1 + w]));
      const float f1 = pow2pos(e1), f2 = pow2pos(e2);
      // state operand fragments (register order over d: K-step s covers c = 32 s ..)
      h8 w1f[2], s1f[2], w2f[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        w1f[st] = tiles_frag(W1s[2 * st], W1s[2 * st + 1], f1);
        s1f[st] = tiles_frag(S1s[2 * st], S1s[2 * st + 1], f1);
        w2f[st] = tiles_frag(W2s[2 * st], W2s[2 * st + 1], f2);
      }
      // W2^T and S2^T copies [u][c] over the workgroup's units (for O and y)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const h8 wf = w2f[ct >> 1];
        const int o = 4 * (ct & 1);
        store_rows4(sW2, RS, uw + lc, 16 * ct + 4 * g, h4{wf[o], wf[o + 1], wf[o + 2], wf[o + 3]});
        store_rows4(sS2, RS, uw + lc, 16 * ct + 4 * g, to_h4(S2s[ct], f2));
      }

      // ================= a2: key-side forward Z1 = K W1^T (rows j, lanes u) =================
      // A1 = SiLU(Z1) and SiLU'(Z1) (fp16, for the backprop).  A1's
      // workgroup-wide operand scale comes from a bound known before the
      // product, so the A1 copy needs no barrier of its own: a sum of 64
      // products gives |Z1[j][u]| <= 64 max|K| max|W1|, and
      // |SiLU(z)| = |z| sigmoid(z) <= |z|.  (Maxima of magnitudes, unlike
      // sums of squares, do not underflow while the state decays.)  The bound
      // may exceed the true maximum by a few binades, which leaves the fp16
      // values normal and rounded exactly as with the exact maximum
      // (power-of-two scaling); a factor 1.001 on the bound covers the fp16
      // rounding of W1.
      int eA1;
      h8 a1f[2];
      f4v SPh[4];   // SiLU'(Z1), fp32
      {
        float mn1 = 0.f, mnk = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
          mn1 = fmaxf(mn1, __int_as_float(ci[INT_N1 + i]));
          mnk = fmaxf(mnk, __int_as_float(ci[INT_NK + i]));
        }
        // 2^-eA1 bounds 64.0641 max|K| max|W1| below 2^14, from the
        // exponents alone (no product that could overflow or underflow)
        eA1 = 0;
        if (mn1 > 0.f && mn1 < INFINITY && mnk > 0.f && mnk < INFINITY) {
          int ea, eb;
          (void)frexpf(mn1, &ea);
          (void)frexpf(mnk, &eb);
          eA1 = 7 - ea - eb;
        }
        const float fA1 = pow2pos(eA1);
        f4v A1f[4];
        const float cx = pow2neg(e1) * -kLog2e;   // Z1 in units of -1/ln 2
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f4v z = {};
          const _Float16* krow = sK + (16 * tt + lc) * RS;
#pragma unroll
          for (int st = 0; st < 2; ++st) z = mfma(frag_rk(krow, 32 * st, g), w1f[st], z);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = z[r] * cx;
            const float sg = sigmoid_x(x);
            const float xs = x * sg;                          // -A1 log2 e
            A1f[tt][r] = xs;
            SPh[tt][r] = fmaf(xs, fmaf(sg, kLn2, -kLn2), sg);   // s + A1 (1 - s) = s (1 + z (1 - s))
          }
        }
        // A1 fragments (register order over the tokens) for the second-layer
        // fold, and the copy [u][j] for O and the scores
#pragma unroll
        for (int st = 0; st < 2; ++st) a1f[st] = tiles_frag(A1f[2 * st], A1f[2 * st + 1], fA1 * -kLn2);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const h8 af = a1f[tt >> 1];
          const int o = 4 * (tt & 1);
          store_rows4(sA1, RS, uw + lc, 16 * tt + 4 * g, h4{af[o], af[o + 1], af[o + 2], af[o + 3]});
        }
      }
      STAMP(4);
      __syncthreads();   // every wave's A1 and W2/S2 copies
      STAMP(5);
      STAMP(6);
      STAMP(7);

      // ================= this workgroup's O = A1 W2^T over its units: tiles (tj, tc0 + i) =================
      float om[kE];
      {
        const float co = pow2neg(eA1 + e2);
#pragma unroll
        for (int i = 0; i < kT; ++i) {
          f4v acc = {};
#pragma unroll
          for (int kk = 0; kk < C::kKSteps; ++kk)
            acc = mfma(frag_tr_c8(sA1, RS, 32 * kk, 16 * tj, g, lc), frag_tr_c8(sW2, RS, 32 * kk, 16 * (tc0 + i), g, lc),
                       acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) om[4 * i + r] = acc[r] * co;
        }
      }
      // publish this workgroup's O (words tagged with this chunk's number)
      const unsigned par = seq & 1u;
#pragma unroll
      for (int e = 0; e < kE / 2; ++e) tstore(xO(h, par), e * kThreads + tid, om[2 * e], om[2 * e + 1], seq);
      unsigned long long* const pub = xP(par) + tid;   // (split) this thread's hand-over words
      float3 g3n;   // (split) the next chunk's gates, token tid (tid < 64)
      STAMP(8);

      // ---- work that does not need the partner, while the exchange is in flight ----
      // this chunk's V for the residual (used after the exchange)
      // Issued unconditionally from a row clamped into the chunk (rows past
      // its end are zeroed at use): a load under a branch would end a basic
      // block and be waited for at once, which also waits for the exchange
      // stores still in flight.
      unsigned short vr[kE];
#pragma unroll
      for (int i = 0; i < kT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = min(16 * tj + 4 * g + r, n - 1);
          vr[4 * i + r] = *(const unsigned short*)(p.v + (tok0 + c0 + j) * kD + 16 * (tc0 + i) + lc);
        }
      const unsigned long long* obases[kG - 1];
#pragma unroll
      for (int m = 0; m < kG - 1; ++m) obases[m] = xO(partner(m), par);
      TPollEarly<kThreads, kE / 2, kG - 1> opoll;
      const bool early_poll = kSplit || w == C::kWD0 || w == C::kWD1;
      // ================= a1: coefficients, while the exchange is in flight =================
      if constexpr (kSplit) {
        key_coef_stage(n);
        opoll.issue(obases, tid);
      } else {
        coef_stage([&] { opoll.issue(obases, tid); });
      }
      // the raw first-layer scores Q K^T (tiles (tj, tc0 + i)) and the query
      // products Q W1^T, Q S1^T
      f4v scr[kT], accW[4], accS[4];
      if constexpr (kRW && !kSplit) raw_scores(scr);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f4v aw = {}, as = {};
        const _Float16* qrow = sQ + (16 * tt + lc) * RS;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const h8 qf = frag_rk(qrow, 32 * st, g);
          aw = mfma(qf, w1f[st], aw);
          if constexpr (kRW) as = mfma(qf, s1f[st], as);
        }
        accW[tt] = aw;
        accS[tt] = as;
      }
      STAMP(9);
      // the partners' O for this thread's elements, and their parts of my y
      // tiles of the previous chunk
      float pvv[kG - 1][kE], pyv[kG - 1][kYPer];
      if (!(early_poll && opoll.check(seq, pvv)) && !tpoll<kThreads, kE / 2, kG - 1>(obases, tid, seq, p.spin_max, pvv))
        give_up();
      if constexpr (!kSplit) {
        if (prev_row0 >= 0) load_prev_y(seq - 1, pyv);
      }
      // every vector memory operation of this thread done, the next chunk's
      // staging loads included (a no-op after a poll, which waited for them)
      __builtin_amdgcn_s_waitcnt(0x0F70);
      STAMP(10);
      // ================= O = the group's partials in workgroup order, Delta2 = O - V =================
      float d2v[kE];
      {
        float am = 0.f, o[kE];
        ordered_sum<kG, kE>(h, om, pvv, o);
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int j = 16 * tj + 4 * g + (e & 3);
          const float vv = __uint_as_float((unsigned)vr[e] << 16);
          d2v[e] = j < n ? o[e] - vv : 0.f;
        }
        am = max_abs(am, d2v);
        am = wave_max(am);
        if (lane == 0) atomicMax((unsigned int*)&ci[INT_AMAX_D2], __float_as_uint(am));
      }
      if constexpr (kSplit) {
        // The retrieval workgroup has read this thread's words of chunk
        // seq - 2 once its receipt carries seq - 2 or seq - 1 (it cannot be
        // further ahead); then the chunk-start W2, S2 copies and A1 go out.
        auto acked = [&](unsigned long long wd) { return tag_is(wd, seq - 2) || tag_is(wd, seq - 1); };
        bool ok = seq <= 2 || acked(ackw);
        for (unsigned it = 0; !ok && it < p.spin_max; ++it) {
          __builtin_amdgcn_s_sleep(1);
          ok = acked(__hip_atomic_load(xA + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        if (!ok) {
          give_up();
        } else {
          // the W2^T and S2^T copies and A1^T in the order of their tiles'
          // 4-value rows (16 each), three values a word, then e2 and eA1
          _Float16 hv[48];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int o = 4 * (ct & 1);
            const h4 sv = to_h4(S2s[ct], f2);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              hv[4 * ct + r] = w2f[ct >> 1][o + r];
              hv[16 + 4 * ct + r] = sv[r];
              hv[32 + 4 * ct + r] = a1f[ct >> 1][o + r];
            }
          }
#pragma unroll
          for (int k = 0; k < 16; ++k)
            wstore(pub + (C::PW_1 + k) * kThreads, h3word(hbits(hv[3 * k]), hbits(hv[3 * k + 1]), hbits(hv[3 * k + 2]), seq));
          wstore(pub + (C::PW_1 + 16) * kThreads, h3word(ebits(e2), ebits(eA1), 0, seq));
        }
        // the next chunk's K and Q into the other tile set (waves 0..3, from
        // their own staging loads, complete since the exchange); its gates
        // wait until every wave is past the coefficient stage
        if (staged) {
          if (w < 4) {
            const float wnk = wave_max(inputs_to_lds(min(p.chunk, p.N - next_c0), tid,
                                                     (_Float16*)(smem + ((seq & 1u) ? OFF_K : OFF_YP)),
                                                     (_Float16*)(smem + ((seq & 1u) ? OFF_Q : OFF_SC)), g3n));
            if (lane == 0) ci[INT_NK + w] = __float_as_int(wnk);
          } else if (lane == 0) {
            ci[INT_NK + w] = 0;   // (max |K| over the pieces of waves 0..3)
          }
        }
      } else {
        // last chunk's y tiles
        if (prev_row0 >= 0) finish_prev_y(pyv);
      }
      STAMP(11);
      __syncthreads();   // every wave's Delta2 amax, the coefficients
      if (ci[INT_FAIL]) { failed = true; break; }
      STAMP(12);
      // the query products' part of Zq1 (diag(A) Q W1^T + diag(F) Q S1^T) in units of -1/ln 2
      const float cz = pow2neg(e1) * -kLog2e;
      auto zq_main = [&](int tt) {
        f4v m;
        if constexpr (kRW) {
          const f4v av = *(const f4v*)(cf + COEF_A + 16 * tt + 4 * g);
          const f4v fv = *(const f4v*)(cf + COEF_F + 16 * tt + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) m[r] = fmaf(av[r], accW[tt][r], fv[r] * accS[tt][r]) * cz;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) m[r] = accW[tt][r] * cz;
        }
        return m;
      };

      // ---- Delta2 (fp16, workgroup-wide scale) as [c][j] ----
      const int eD2 = scale_exp(__uint_as_float((unsigned)ci[INT_AMAX_D2]));
      {
        const float fD2 = pow2pos(eD2);
        h4 hv[kT];
#pragma unroll
        for (int i = 0; i < kT; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[i][r] = sc16(d2v[4 * i + r], fD2);
          *(h4*)(sD2T + (16 * (tc0 + i) + lc) * RS + 16 * tj + 4 * g) = hv[i];
        }
        if constexpr (kSplit) {
          // Delta2 (8 values) and eD2 in three words, then the query
          // products (eight twords)
          static_assert(kT == 2, "eight Delta2 values a thread");
          wstore(pub + (C::PW_2 + 0) * kThreads, h3word(hbits(hv[0][0]), hbits(hv[0][1]), hbits(hv[0][2]), seq));
          wstore(pub + (C::PW_2 + 1) * kThreads, h3word(hbits(hv[0][3]), hbits(hv[1][0]), hbits(hv[1][1]), seq));
          wstore(pub + (C::PW_2 + 2) * kThreads, h3word(hbits(hv[1][2]), hbits(hv[1][3]), ebits(eD2), seq));
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const f4v m = zq_main(tt);
            wstore(pub + (C::PW_2 + 3 + 2 * tt) * kThreads, tword(m[0], m[1], seq));
            wstore(pub + (C::PW_2 + 4 + 2 * tt) * kThreads, tword(m[2], m[3], seq));
          }
        }
      }
      if constexpr (kRW && !kSplit) sc1_store(scr);
      if constexpr (kSplit) {
        if (staged && w == 0) gates_to_lds(tid, g3n);
      }
      if (!kSplit && w == C::kWD0) {
        // weights of the state update: U_i = theta_i prod_{m>i} eta_m and
        // D[n-1][i] (padding has eta = 1)
        const int i = lane;
        const float ti = cf[COEF_XT + i];
        store_fold_weights(i, i < 32 ? ti * __int_as_float(ci[INT_T22]) : ti, d_full(n - 1, i));
      }
      STAMP(13);
      __syncthreads();   // Delta2 copies, the first-layer scores and the update weights
      STAMP(14);

      // ================= a3: Delta1 = (Delta2 W2) * SiLU'(Z1)  (rows j, lanes u) =================
      h8 d1f[2];
      int eD1;
      {
        f4v Df[4];
        float am = 0.f;
        const float dun = pow2neg(eD2 + e2);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f4v acc = {};
#pragma unroll
          for (int st = 0; st < 2; ++st) acc = mfma(frag_tr_rk(sD2T, RS, 32 * st, 16 * tt, g, lc), w2f[st], acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) Df[tt][r] = acc[r] * dun * SPh[tt][r];
          am = max4(am, Df[tt]);
        }
        eD1 = scale_exp(wave_max(am));
        const float fD1 = pow2pos(eD1);
#pragma unroll
        for (int st = 0; st < 2; ++st) d1f[st] = tiles_frag(Df[2 * st], Df[2 * st + 1], fD1);
      }
      if constexpr (kSplit) {
        // Delta1's fragments (16 values) and eD1 in six words
        unsigned short hv[18];
#pragma unroll
        for (int e = 0; e < 16; ++e) hv[e] = hbits(d1f[e >> 3][e & 7]);
        hv[16] = ebits(eD1);
        hv[17] = 0;
#pragma unroll
        for (int k = 0; k < 6; ++k)
          wstore(pub + (C::PW_3 + k) * kThreads, h3word(hv[3 * k], hv[3 * k + 1], hv[3 * k + 2], seq));
      }

      STAMP(15);
      f4v H1f[4];
      if constexpr (!kSplit) zq1_h1(zq_main, d1f, eD1, H1f);

      STAMP(16);
      const float An = cf[COEF_A + n - 1], En = cf[COEF_E + n - 1], Fn = cf[COEF_F + n - 1];
      const int ewU = ci[INT_EWU], ewD = ci[INT_EWD];
      float m1n = 0.f, m2n = 0.f, n1n = 0.f;   // the new state's maxima of |S1|, |W2| and |S2|, |W1|
      // the fold weights as fragments in register order over the tokens
      h8 wuf[2], wdf[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        wuf[st] = frag_rk(ch + H16_WU, 32 * st, g);
        wdf[st] = frag_rk(ch + H16_WD, 32 * st, g);
      }
      // ================= a4, layer 1 (W1, S1 are not read again this chunk) =================
      // G1^T[c][u] = sum_j K[j][c] w_j Delta1[j][u]
      {
        const float uD1 = pow2neg(ewD + eD1), uU1 = pow2neg(ewU + eD1);
        const h8 bu0 = d1f[0] * wuf[0], bu1 = d1f[1] * wuf[1];
        const h8 bd0 = d1f[0] * wdf[0], bd1 = d1f[1] * wdf[1];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const h8 k0 = frag_tr_rk(sK, RS, 0, 16 * ct, g, lc), k1 = frag_tr_rk(sK, RS, 32, 16 * ct, g, lc);
          f4v gU = {}, gD = {};
          gU = mfma(k0, bu0, gU);
          gU = mfma(k1, bu1, gU);
          gD = mfma(k0, bd0, gD);
          gD = mfma(k1, bd1, gD);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float w0 = W1s[ct][r], s0 = S1s[ct][r];
            W1s[ct][r] = fmaf(gD[r], -uD1, fmaf(An, w0, Fn * s0));
            S1s[ct][r] = fmaf(gU[r], -uU1, En * s0);
          }
          n1n = max4(n1n, W1s[ct]);
          m1n = max4(m1n, S1s[ct]);
        }
      }
      STAMP(17);
      int eH1 = 0;
      if constexpr (!kSplit) {
        __syncthreads();   // every wave's H1 maximum
        eH1 = h1_copy(H1f);
      }
      STAMP(18);
      if constexpr (!kSplit) __syncthreads();   // every wave's H1 copy
      STAMP(19);
      if constexpr (kRW && !kSplit) p_scores(eH1, eA1);

      STAMP(20);
      // ================= a4, layer 2: G2^T[c][u] = sum_j Delta2[j][c] w_j A1[j][u] =================
      {
        const float uD2 = pow2neg(ewD + eA1 + eD2), uU2 = pow2neg(ewU + eA1 + eD2);
        const h8 bu0 = a1f[0] * wuf[0], bu1 = a1f[1] * wuf[1];
        const h8 bd0 = a1f[0] * wdf[0], bd1 = a1f[1] * wdf[1];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const _Float16* arow = sD2T + (16 * ct + lc) * RS;
          const h8 d0 = frag_rk(arow, 0, g), d1 = frag_rk(arow, 32, g);
          f4v gU = {}, gD = {};
          gU = mfma(d0, bu0, gU);
          gU = mfma(d1, bu1, gU);
          gD = mfma(d0, bd0, gD);
          gD = mfma(d1, bd1, gD);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float w0 = W2s[ct][r], s0 = S2s[ct][r];
            W2s[ct][r] = fmaf(gD[r], -uD2, fmaf(An, w0, Fn * s0));
            S2s[ct][r] = fmaf(gU[r], -uU2, En * s0);
          }
          m2n = max4(max4(m2n, W2s[ct]), S2s[ct]);
        }
      }
      STAMP(21);
      if constexpr (!kSplit) {
        __syncthreads();   // every wave's second-layer scores
        y_stage(eH1, e2, eD2, par);
      }
      // the new state's maxima for the next chunk's operand scales (reduced
      // here, once the fold's products have long completed)
      {
        const float wn1 = wave_max(n1n), wm1 = fmaxf(wave_max(m1n), wn1), wm2 = wave_max(m2n);
        if (lane == 0) {
          ci[INT_M1 + w] = __float_as_int(wm1);
          ci[INT_N1 + w] = __float_as_int(wn1);
          ci[INT_M2 + w] = __float_as_int(wm2);
        }
      }
      if constexpr (early) {
        // the next chunk's inputs into their tiles (waves 4..7, beside y on
        // waves 0..3), then the chunk after it into the staging area
        if (staged) {
          if (w >= 4) {
            const int nn = min(p.chunk, p.N - next_c0);
            float3 g3;
            const float wnk = wave_max(inputs_to_lds(nn, tid - 256, sK, sQ, g3));
            gates_to_lds(tid - 256, g3);
            if (lane == 0) ci[INT_NK + w] = __float_as_int(wnk);
            int s2 = next_s, c2 = next_c0 + p.chunk, i2 = next_ci + 1;
            if (c2 >= p.N) { s2 = next_s + p.n_groups; c2 = 0; i2 = 0; }
            if (s2 < p.streams) {
              // this thread's staging reads are complete before the slots it
              // read are refilled (the same threads refill them)
              __builtin_amdgcn_s_waitcnt(0xC07F);
              prefetch_chunk_lds<256>(p, (int64_t)s2 * p.N + c2, gate_base(p, s2, i2, c2), min(p.chunk, p.N - c2),
                                      tid - 256, smem + OFF_STAGE);
            }
          } else if (lane == 0) {
            ci[INT_NK + w] = 0;   // (max |K| over the slots of waves 4..7)
          }
        }
        pre = staged;
        if (staged) {
          int s2 = next_s, c2 = next_c0 + p.chunk;
          if (c2 >= p.N) { s2 = next_s + p.n_groups; c2 = 0; }
          staged = s2 < p.streams;
        }
      }
      if constexpr (kSplit) pre = staged;
      STAMP(22);
      prev_row0 = tok0 + c0;
      prev_n = n;
      __syncthreads();   // LDS tiles are rewritten by the next chunk
      STAMP(23);
    }

    if (failed) break;
    if constexpr (kSplit) {
      // The retrieval workgroup has read the stream's last words before the
      // state goes out: a give-up of it until then (which poisons the
      // stream's outputs) never precedes this write.
      bool ok = tag_is(__hip_atomic_load(xA + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), seq);
      for (unsigned it = 0; !ok && it < p.spin_max; ++it) {
        __builtin_amdgcn_s_sleep(1);
        ok = tag_is(__hip_atomic_load(xA + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), seq);
      }
      if (!ok) give_up();
      __syncthreads();
      if (ci[INT_FAIL]) { failed = true; break; }
    }
    // ---- write this wave's part of the final state ----
    {
      float* Wo = p.W_out + (int64_t)s * kP;
      float* So = p.S_out + (int64_t)s * kP;
      const int u = hs + lc;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = 16 * ct + 4 * g;
        *(f4v*)(Wo + u * kD + c) = W1s[ct];
        *(f4v*)(So + u * kD + c) = S1s[ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Wo[kH * kD + (c + r) * kH + u] = W2s[ct][r];
          So[kH * kD + (c + r) * kH + u] = S2s[ct][r];
        }
      }
    }
  }

  // the last chunk's y rows
  if (!kSplit && !failed && prev_row0 >= 0) {
    float pyv[kG - 1][kYPer];
    load_prev_y(seq, pyv);
    finish_prev_y(pyv);   // (rows of a wait that gave up are overwritten below)
    __syncthreads();
    if (ci[INT_FAIL]) failed = true;
  }
  if (failed) poison_group_streams<kThreads>(p, grp, tid);
  // no load into this workgroup's LDS may outlive it (a workgroup that gave up
  // can leave a staging prefetch in flight)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace

bool mlp2_supported(const Shape& s, int chunk) {
  return s.L == 2 && s.d == kD && s.hidden == kH && s.io == TM_IO_BF16 &&
         (s.read_mode == TM_READ_AFTER_WRITE || s.read_mode == TM_READ_CHUNK_START) && chunk >= 1 && chunk <= kB;
}

// Eight waves per workgroup for every stream count: four-wave workgroups
// in groups of four (a few streams over twice as many CUs) measured slower
// per chunk, since a chunk's time is each wave's own dependency chain and
// a four-wave workgroup's waves carry twice the workgroup-level tiles.
using GrpUsed = Grp<8>;
static int64_t groups_for(const Shape& s) {
  return s.streams < GrpUsed::kMaxGroups ? s.streams : GrpUsed::kMaxGroups;
}
// With few streams (at most a quarter as many as a 256-CU device has CUs)
// and retrieval after each write, each half's retrieval runs on a workgroup
// of its own (kSplit), four workgroups per stream, when the device holds
// them all at once; the workspace then also holds the hand-over words.
static bool split_shape(const Shape& s) {
  return s.read_mode == TM_READ_AFTER_WRITE && s.streams <= GrpUsed::kMaxGroupsSplit;
}
static int64_t group_bytes(const Shape& s) {
  return split_shape(s) ? GrpUsed::kGroupBytesSplit : GrpUsed::kGroupBytes;
}

int64_t mlp2_ws_bytes(const Shape& s, int) { return groups_for(s) * group_bytes(s) + 256; }

int64_t mlp2_status_offset(const Shape& s) { return groups_for(s) * group_bytes(s); }

// ---- scratch of titans_mem_forward_noalloc ----
// The kernel's workspace (exchange buffers and status word) for the
// largest group count, as a file-scope device array: one copy per GPU,
// allocated when the library's code object is loaded on that device and
// held until the process ends.  Host code must not use the array's name as
// an address: its device address is looked up once per device with
// hipGetSymbolAddress and kept below.  Every call on one GPU shares the
// array; every call clears the exchange buffers and the status word with a
// fill kernel (no memset) before the memory kernel, so calls that follow one
// another are independent, while calls that overlap on one GPU race.
constexpr int64_t kScratchBytes =
    (GrpUsed::kMaxGroups * GrpUsed::kGroupBytes > GrpUsed::kMaxGroupsSplit * GrpUsed::kGroupBytesSplit
         ? GrpUsed::kMaxGroups * GrpUsed::kGroupBytes
         : GrpUsed::kMaxGroupsSplit * GrpUsed::kGroupBytesSplit) +
    256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // per device: the device address of `scratch`, once looked up
}  // namespace

int64_t mlp2_scratch_bytes() { return kScratchBytes; }

hipError_t mlp2_scratch(void** out, bool lookup) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev] && lookup) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

#if TM_STAGE_STAMPS
}  // namespace titans
extern "C" int titans_mem_stage_stamps(unsigned long long* dst, int64_t count) {
  if (count > (int64_t)titans::kStampChunks * titans::kMaxWaves * titans::kStampStages) return TM_ERR_INVALID;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(titans::stage_stamps), count * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? TM_OK : TM_ERR_HIP;
}
namespace titans {
#endif

template <int NW>
static hipError_t launch_group(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                               const float* alpha, const float* eta, const float* theta, const float* W_in,
                               const float* S_in, void* y, float* W_out, float* S_out, void* ws,
                               hipStream_t stream) {
  using C = Grp<NW>;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // every group must be resident at once (one workgroup per CU)
  int64_t ng = groups_for(s);
  if (ng > cus / C::kG) ng = cus / C::kG;
  if (ng < 1) return hipErrorInvalidConfiguration;
  const bool rw = s.read_mode == TM_READ_AFTER_WRITE;
  // the retrieval on workgroups of its own while every group's four fit at once
  const bool split = NW == 8 && split_shape(s) && 2 * C::kG * ng <= cus;
  // otherwise each chunk's inputs moved into LDS during the previous chunk
  // only while at most half the CUs run a workgroup: 2% faster with few
  // streams, 1% slower with every CU busy
  const bool early = !split && NW == 8 && 2 * C::kG * ng <= cus;
  const void* kfn = rw ? (early ? (const void*)mlp2_group_kernel<true, NW, true, false>
                                : (const void*)mlp2_group_kernel<true, NW, false, false>)
                       : (early ? (const void*)mlp2_group_kernel<false, NW, true, false>
                                : (const void*)mlp2_group_kernel<false, NW, false, false>);
  if constexpr (NW == 8)
    if (split) kfn = (const void*)mlp2_group_kernel<true, NW, false, true>;
  // the kernel's dynamic LDS size, set on every call (no state kept between
  // calls; idempotent and cheap next to the kernel)
  e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
  if (e != hipSuccess) return e;
  Params p;
  p.N = s.N;
  p.chunk = chunk;
  p.streams = s.streams;
  p.n_groups = (int)ng;
  p.k = (const __hip_bfloat16*)k;
  p.v = (const __hip_bfloat16*)v;
  p.q = (const __hip_bfloat16*)q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.W_in = W_in;
  p.S_in = S_in;
  p.y = (__hip_bfloat16*)y;
  p.W_out = W_out;
  p.S_out = S_out;
  unsigned char* base = (unsigned char*)ws;
  p.xbuf = base;
  p.status = (unsigned*)(base + mlp2_status_offset(s));
  p.spin_max = (s.flags & TM_FLAG_NO_WAIT) ? 0u : kSpinMax;
  p.chunk_gates = s.chunk_gates;
  p.gstride = s.chunk_gates ? (s.N + chunk - 1) / chunk : s.N;
  const int64_t n16 = ng * (split ? C::kGroupBytesSplit : C::kGroupBytes) / 16;
  hipLaunchKernelGGL(zero_exchange_kernel, dim3((unsigned)std::min<int64_t>((n16 + 255) / 256, 1024)), dim3(256), 0,
                     stream, (uint4*)base, n16, p.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((split ? 2 : 1) * C::kG * ng)), block(C::kThreads);
  if (split) {
    if constexpr (NW == 8)
      hipLaunchKernelGGL((mlp2_group_kernel<true, NW, false, true>), grid, block, C::kLdsBytes, stream, p);
  } else if (rw && early) {
    hipLaunchKernelGGL((mlp2_group_kernel<true, NW, true, false>), grid, block, C::kLdsBytes, stream, p);
  } else if (rw) {
    hipLaunchKernelGGL((mlp2_group_kernel<true, NW, false, false>), grid, block, C::kLdsBytes, stream, p);
  } else if (early) {
    hipLaunchKernelGGL((mlp2_group_kernel<false, NW, true, false>), grid, block, C::kLdsBytes, stream, p);
  } else {
    hipLaunchKernelGGL((mlp2_group_kernel<false, NW, false, false>), grid, block, C::kLdsBytes, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_mlp2(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                       const float* alpha, const float* eta, const float* theta,
                       const float* W_in, const float* S_in, void* y, float* W_out,
                       float* S_out, void* ws, hipStream_t stream) {
  return launch_group<GrpUsed::kWaves>(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y, W_out, S_out, ws,
                                       stream);
}

}  // namespace titans
