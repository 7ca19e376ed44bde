// Specialised MFMA kernel: 2-layer memory, d = 64, hidden = 256, chunk <= 64,
// bf16 keys/values/queries/outputs, fp32 state and gates.
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
//   half of the hidden layer; each workgroup is 4 waves (one per SIMD) and
//   wave w owns 32 hidden units.  Everything per hidden unit (the state rows
//   and columns, A1, Delta1, H1, the state update) is local to its wave.
//   Only the two contractions over all 256 hidden units cross the pair: O
//   (needed before the backprop: one exchange per chunk on the critical
//   path) and y (exchanged one chunk late, riding on the next O exchange).
//   With 128 streams this fills all 256 CUs, and it halves the state each
//   CU must hold.
// * The fp32 state of a wave (W1, S1, W2, S2 restricted to its 32 hidden
//   units: 4 x 64 x 32 floats) lives in accumulation registers (AGPRs) for
//   the whole sequence, in the accumulator layout of
//   v_mfma_f32_32x32x16_f16: the update GEMMs land in that layout, and an
//   accumulator tile (lane = column, registers = rows) feeds the next MFMA
//   as an operand contracting over its rows, so the state is used as an
//   MFMA operand without an LDS round trip (only W2 needs one transposed
//   copy per chunk, for the backprop).
// * Every MFMA operand is fp16 with a power-of-two scale per operand block
//   and chunk (fp32 accumulation, exact rescaling).  bf16 operands lose
//   about 1e-2 relative on the state; scaled fp16 keeps about 1e-3.
// * The pair exchanges partial sums through global memory with agent-
//   coherent (sc1) relaxed accesses: data stores, s_waitcnt vmcnt(0), then a
//   sequence flag; the reader polls the flag with a bounded spin.  A pair
//   whose partner never arrives gives up, writes NaN to its stream's state
//   and records the failure in the workspace status word.  Sums are formed
//   in a fixed order (half 0 + half 1), so results are bitwise reproducible
//   and identical in both halves.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

namespace titans {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kD = 64;
constexpr int kH = 256;
constexpr int kB = 64;           // token rows per chunk tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHW = 32;          // hidden units per wave
constexpr int kHC = kWaves * kHW;  // hidden units per workgroup (half of kH)
constexpr int kP = 2 * kD * kH;
constexpr int RS = 68;           // fp16 row stride (halves) of 64-wide tiles
constexpr int RSA = 36;          // fp16 row stride of the 32-wide A1 copy
constexpr int RSF = 68;          // fp32 row stride (floats)
constexpr int kMaxPairs = 128;
constexpr unsigned kSpinMax = 1u << 21;

// ---- LDS layout (bytes) ----
constexpr int kTileH = kB * RS * 2;                  // 64 x 68 fp16 = 8704
constexpr int OFF_K = 0;
constexpr int OFF_KT = OFF_K + kTileH;
constexpr int OFF_Q = OFF_KT + kTileH;
constexpr int OFF_D2 = OFF_Q + kTileH;
constexpr int OFF_D2T = OFF_D2 + kTileH;
constexpr int OFF_SC1 = OFF_D2T + kTileH;
constexpr int OFF_DM = OFF_SC1 + kTileH;             // fp32 [64][68]
constexpr int OFF_COEF = OFF_DM + kB * RSF * 4;
// float index: XT = the D recurrences' carried products (see the a1 stage),
// T11/T12 = transfer of rows 32..63 (32 entries each)
constexpr int COEF_XT = 0, COEF_T11 = 64, COEF_T12 = 96, COEF_THETA = 128, COEF_A = 192, COEF_E = 256,
              COEF_F = 320;
constexpr int COEF_H16 = 512 * 4;                                   // byte offset of fp16 arrays
constexpr int H16_WU = 128, H16_WD = 192;                           // half index
constexpr int COEF_INT = COEF_H16 + 256 * 2;                        // byte offset of int slots
constexpr int COEF_PAIR = COEF_INT + 16 * 4;                        // byte offset of (1-alpha, eta) pairs
constexpr int kCoefBytes = COEF_PAIR + kB * 8;
constexpr int OFF_WAVE = (OFF_COEF + kCoefBytes + 255) / 256 * 256;
// per-wave region: [A1 copy 64 x RSA fp16][W2 copy [h_l][c] 32 x RS fp16][W2 copy [c][h_l] 64 x RSA fp16];
// later the whole region holds the wave's y partial (64 x RSF fp32, token-major)
constexpr int kA1Bytes = kB * RSA * 2;               // 4608
constexpr int kW2Bytes = kHW * RS * 2;               // 4352: W2 copy [h_l][c]
constexpr int kWaveRegion = kD * RSF * 4;            // 17408
// staging for the next chunk's raw bf16 K, Q rows and gates (filled during the
// pair handshake, converted at the next chunk's start)
constexpr int OFF_STAGE = OFF_WAVE + kWaves * kWaveRegion;
constexpr int kStageBytes = 2 * kB * kD * 2 + 3 * kB * 4;
constexpr int kLdsBytes = OFF_STAGE + kStageBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kA1Bytes + kW2Bytes + kD * RSA * 2 <= kWaveRegion, "A1 copy + both W2 copies");

constexpr int INT_AMAX_SC1 = 0, INT_AMAX_D2 = 1, INT_EWU = 2, INT_EWD = 3, INT_FAIL = 4, INT_T22 = 5;
constexpr int INT_M2 = 6, INT_MA1 = 10;   // per-wave maxima (4 slots each) for the workgroup-wide scales

// ---- global workspace layout, per pair (bytes) ----
constexpr int64_t kXO = 2 * 2 * kB * kD * 4;         // [half][parity] x 64 x 64 fp32, thread-major
constexpr int64_t kXY = 2 * 2 * 32 * kD * 4;         // [half][parity] x 32 x 64 fp32, thread-major
constexpr int64_t kPairBytes = kXO + kXY;
constexpr int64_t kFlagStride = 128;                  // bytes between flags (own cache line)

struct Params {
  int N, chunk, streams, n_pairs;
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
  unsigned char* xbuf;   // n_pairs * kPairBytes
  unsigned* flags;       // n_pairs * 2 flags, kFlagStride apart
  unsigned* status;      // set to 1 when a pair gave up waiting
  unsigned spin_max;
  int chunk_gates;       // gates hold one value per chunk
};

// index of token t0's gate, and the step per following token of the chunk
__device__ __forceinline__ int64_t gate_base(const Params& p, int s, int c0) {
  return p.chunk_gates ? (int64_t)s * ((p.N + p.chunk - 1) / p.chunk) + c0 / p.chunk : (int64_t)s * p.N + c0;
}

// accumulator row of register r for lane group lg (32x32 tile)
__device__ __forceinline__ int crow(int r, int lg) { return 8 * (r >> 2) + 4 * lg + (r & 3); }

__device__ __forceinline__ f16v mfma(h8 a, h8 b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 fp16 operand values of one lane for K-step s of a 32-wide block at
// column kbase of an LDS row: contraction slots follow the accumulator row
// order (two runs of 4: kbase+4lg.. and kbase+8+4lg..).
__device__ __forceinline__ h8 lds_frag(const _Float16* row, int kbase, int lg) {
  h4 lo = *(const h4*)(row + kbase + 4 * lg);
  h4 hi = *(const h4*)(row + kbase + 8 + 4 * lg);
  return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ h8 hmul(h8 a, h8 b) { return a * b; }

// The fp32 state lives in accumulation registers (AGPRs); VALU reaches it
// only through these moves, which keeps the architectural VGPRs for the
// chunk's working set.  They are plain register moves (not volatile), so
// the scheduler may place them freely.
__device__ __forceinline__ float ag_get(float a) {
  float v;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}
__device__ __forceinline__ float ag_put(float v) {
  float a;
  asm("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}
struct Tile {   // one 32x32 fp32 accumulator tile of the state
  float r[16];
};

__device__ __forceinline__ h8 state_frag(const Tile& t, int s, float fe) {
  h8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)(ag_get(t.r[8 * s + i]) * fe);
  return r;
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

// maximum over the wave, returned uniformly
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));   // every lane of a row of 16 holds the row's maximum
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
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

// 2^-k as a float multiplier: exact rescaling (same result as ldexpf(x, -k))
// while 2^-k is a normal float, i.e. k <= 126; beyond that the factor
// flushes towards zero (scaled values far below any tolerance floor).  k is
// clamped below so that the factor stays finite.
__device__ __forceinline__ float pow2neg(int k) { return ldexpf(1.f, -max(k, -126)); }
// 2^e as a float multiplier for the scalings up to fp16 operands (one
// multiply per element instead of an ldexp; computed once per block).  Equal
// to ldexpf(x, e) whenever e <= 127, i.e. unless the block's amax is below
// 2^-113, where the clamped scale leaves the operand smaller than [2^13, 2^14)
// but still far below every tolerance floor.
__device__ __forceinline__ float pow2pos(int e) { return ldexpf(1.f, min(e, 127)); }

// per-token factors of the retrieval operands: (A_j, F_j) scaled by a
// common power of two 2^s so that the larger lies in (0.5, 1] (fp16 keeps
// both with 11 significant bits); s is returned for the unscaling
__device__ __forceinline__ void token_factors(float a, float f, _Float16& ah, _Float16& fh, int& s) {
  const float m = fmaxf(fabsf(a), fabsf(f));
  int e = 0;
  if (m > 0.f && m < INFINITY) (void)frexpf(m, &e);
  s = -e;
  ah = (_Float16)ldexpf(a, s);
  fh = (_Float16)ldexpf(f, s);
}
__device__ __forceinline__ h8 hscale(h8 x, _Float16 c) { return x * c; }

__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Pair exchange accessors: agent-coherent (sc1) relaxed accesses, ordered by
// s_waitcnt vmcnt(0) before each flag store.  (L2-local variants for halves
// on one XCD -- workgroup-scope stores and loads, with or without dropping
// the reader's L1 lines before each poll -- left a poller reading a stale
// flag on gfx950, so the exchange stays agent-coherent.)
// The exchange buffers are thread-major: 8-byte element e of thread t sits
// at (e * kThreads + t) * 8 bytes, so each store or load instruction of a
// wave covers 512 contiguous bytes (whole lines: an agent-coherent store
// writes through L2, and scattered 8-byte pieces would each cost a sector).
// Every thread reads back exactly the elements the same thread of the
// partner wrote.
__device__ __forceinline__ void xstore2(float* base, int e, int t, float a, float b) {
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store((unsigned long long*)base + (e * kThreads + t), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 8 floats = elements e0 .. e0+3 of thread t
__device__ __forceinline__ void xload8(const float* base, int e0, int t, float* a) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned long long v = __hip_atomic_load((const unsigned long long*)base + ((e0 + i) * kThreads + t),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a[2 * i] = __uint_as_float((unsigned)v);
    a[2 * i + 1] = __uint_as_float((unsigned)(v >> 32));
  }
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// A flag read through the XCD's L2: a scalar load that bypasses the scalar
// cache (glc).  Valid when the writer runs on the same XCD, whose stores pass
// through that L2; a writer on another XCD could leave a stale L2 line, so the
// caller uses it only after checking that both halves share an XCD.
__device__ __forceinline__ unsigned load_flag_l2(const unsigned* f) {
  unsigned v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(f) : "memory");
  return v;
}

// one thread's share of a chunk's raw inputs: 16 bf16 of a K row and of a Q
// row (row j = tid/4, columns (tid%4)*16..), and for tid < 64 the gates of
// token tid; rows and tokens past the chunk end read as zeros (gates as
// "no forgetting, no decay, no write")
struct ChunkRegs {
  uint4 k0, k1, q0, q1;
  float ga, ge, gt;
};

__device__ __forceinline__ ChunkRegs load_chunk_regs(const Params& p, int64_t row0, int64_t g0, int n, int tid) {
  ChunkRegs r;
  const int j = tid >> 2, cb = (tid & 3) * 16;
  if (j < n) {
    const uint4* kr = (const uint4*)(p.k + (row0 + j) * kD + cb);
    const uint4* qr = (const uint4*)(p.q + (row0 + j) * kD + cb);
    r.k0 = kr[0]; r.k1 = kr[1]; r.q0 = qr[0]; r.q1 = qr[1];
  } else {
    r.k0 = r.k1 = r.q0 = r.q1 = make_uint4(0, 0, 0, 0);
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
// or 4 bytes at base + 4 l; lanes that do not load write nothing).  Thread
// t = 64 w + l loads the same 32 bytes of a K and a Q row that
// load_chunk_regs gives it: slot (2w + i) * 64 + l of each area holds its
// i-th 16 bytes.  Wave 0 loads the gates.  Rows and tokens past the chunk end
// are left out and replaced on unstaging.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ void prefetch_chunk_lds(const Params& p, int64_t row0, int64_t g0, int n, int tid,
                                                   unsigned char* stage) {
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = tid >> 2, cb = (tid & 3) * 16;
  uint4* sk = (uint4*)stage;
  uint4* sq = (uint4*)(stage + kB * kD * 2);
  if (j < n) {
    const uint4* kr = (const uint4*)(p.k + (row0 + j) * kD + cb);
    const uint4* qr = (const uint4*)(p.q + (row0 + j) * kD + cb);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(kr + i), (lds_void_ptr)(sk + (2 * w + i) * 64), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(qr + i), (lds_void_ptr)(sq + (2 * w + i) * 64), 16, 0, 0);
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

__device__ __forceinline__ ChunkRegs unstage_chunk_regs(const unsigned char* stage, int n, int tid) {
  ChunkRegs r;
  const int w = tid >> 6, lane = tid & 63, j = tid >> 2;
  const uint4* sk = (const uint4*)stage;
  const uint4* sq = (const uint4*)(stage + kB * kD * 2);
  if (j < n) {
    r.k0 = sk[(2 * w) * 64 + lane]; r.k1 = sk[(2 * w + 1) * 64 + lane];
    r.q0 = sq[(2 * w) * 64 + lane]; r.q1 = sq[(2 * w + 1) * 64 + lane];
  } else {
    r.k0 = r.k1 = r.q0 = r.q1 = make_uint4(0, 0, 0, 0);
  }
  r.ga = 0.f; r.ge = 1.f; r.gt = 0.f;
  if (tid < kB && tid < n) {
    const float* g = (const float*)(stage + 2 * kB * kD * 2);
    r.ga = g[tid]; r.ge = g[kB + tid]; r.gt = g[2 * kB + tid];
  }
  return r;
}

__device__ __forceinline__ void bf16x8_to_h(const uint4 u, _Float16* out) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xffff0000u);
  }
}

__global__ void zero_flags_kernel(unsigned* flags, int n, unsigned* status) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    flags[(int64_t)i * (kFlagStride / 4)] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0u;
}

// kRW: retrieval after each token's write (true) or at the chunk-start
// state (false: y_j = M_{W_0}(q_j), without the masked correction terms)
template <bool kRW>
__global__ void __launch_bounds__(kThreads, 1) mlp2_pair_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* sK = (_Float16*)(smem + OFF_K);
  _Float16* sKT = (_Float16*)(smem + OFF_KT);
  _Float16* sQ = (_Float16*)(smem + OFF_Q);
  _Float16* sD2 = (_Float16*)(smem + OFF_D2);
  _Float16* sD2T = (_Float16*)(smem + OFF_D2T);
  _Float16* sSC1 = (_Float16*)(smem + OFF_SC1);
  float* sDM = (float*)(smem + OFF_DM);
  float* cf = (float*)(smem + OFF_COEF);
  _Float16* ch = (_Float16*)(smem + OFF_COEF + COEF_H16);
  int* ci = (int*)(smem + OFF_COEF + COEF_INT);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lg = lane >> 5;

  // pair / half: blocks g and g + 8 usually share an XCD (round-robin dispatch),
  // so pairs are formed that way when the grid allows it; correctness does
  // not depend on the placement
  int pair, half;
  {
    const int g = blockIdx.x;
    if ((gridDim.x & 15) == 0) {
      const int slot = g >> 3;
      pair = (g & 7) + 8 * (slot >> 1);
      half = slot & 1;
    } else {
      pair = g >> 1;
      half = g & 1;
    }
  }
  const int hs = kHC * half + kHW * w;   // first hidden unit of this wave
  _Float16* sRA = (_Float16*)(smem + OFF_WAVE + w * kWaveRegion);       // A1 copy [j][h_l]
  _Float16* sRW = (_Float16*)(smem + OFF_WAVE + w * kWaveRegion + kA1Bytes);  // W2 copy [h_l][c]
  _Float16* sRW2 = (_Float16*)(smem + OFF_WAVE + w * kWaveRegion + kA1Bytes + kW2Bytes);   // W2 copy [c][h_l]
  float* sRF = (float*)(smem + OFF_WAVE + w * kWaveRegion);              // y partial [j][c]

  unsigned char* xb = p.xbuf + (int64_t)pair * kPairBytes;
  float* xO_me = (float*)(xb) + half * 2 * kB * kD;
  const float* xO_pt = (const float*)(xb) + (1 - half) * 2 * kB * kD;
  float* xY_me = (float*)(xb + kXO) + half * 2 * 32 * kD;
  const float* xY_pt = (const float*)(xb + kXO) + (1 - half) * 2 * 32 * kD;
  bool failed0 = false;
  unsigned* flag_me = p.flags + (int64_t)(2 * pair + half) * (kFlagStride / 4);
  const unsigned* flag_pt = p.flags + (int64_t)(2 * pair + 1 - half) * (kFlagStride / 4);

  // pair handshake: publish `seq`, then every thread runs `first` (loads
  // that must not delay the flag: the flag waits for this wave's earlier
  // memory operations, loads included), then waves 1..3 run `during` while
  // thread 0 waits for the partner's `seq`; false = gave up
  bool same_xcd = false;   // set after the first handshake (which polls through memory)
  auto handshake = [&](unsigned seq, auto&& first, auto&& during) -> bool {
    wait_stores();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flag_me, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    first();
    if (tid == 0) {
      unsigned it = 0;
      if (same_xcd) {
        while (load_flag_l2(flag_pt) < seq) {
          if (++it >= p.spin_max) break;
          __builtin_amdgcn_s_sleep(1);
        }
      } else {
        while (__hip_atomic_load(flag_pt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < seq) {
          if (++it >= p.spin_max) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      const int ok = it < p.spin_max;
      if (!ok) __hip_atomic_store(p.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ci[INT_FAIL] = ok ? 0 : 1;
    } else {
      during();
    }
    __syncthreads();
    return ci[INT_FAIL] == 0;
  };
  auto nothing = [] {};

  // the pair starts together, polling through memory; each half also
  // publishes the XCD it runs on (before its flag), and when the two agree
  // the later polls read the flag through the shared L2
  const unsigned xcc_me = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xfu;   // HW_REG_XCC_ID
  if (tid == 0) __hip_atomic_store(flag_me + 1, xcc_me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!handshake(1u, nothing, nothing)) failed0 = true;
  same_xcd = __builtin_amdgcn_readfirstlane(
                 __hip_atomic_load(flag_pt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == xcc_me ? 1 : 0) != 0;

  // my y rows of the previous chunk, kept across the chunk boundary:
  // thread t covers row j = 32*half + t/8, columns (t%8)*8 .. +8
  float ymine[8];
  int64_t prev_row0 = -1;   // global token row of the previous chunk's first token
  int prev_n = 0;
  unsigned seq = 0;
  bool failed = failed0;
  bool staged = false;   // the staging area holds the rows of the chunk about to start

  // the partner's partial for my rows of the previous chunk (thread-major)
  auto load_prev_y = [&](unsigned parity, float* pv) { xload8(xY_pt + parity * 32 * kD, 0, tid, pv); };
  // the fixed-order sum of the two partials, stored as bf16
  auto finish_prev_y = [&](const float* pv) {
    const int jr = tid >> 3, cc = (tid & 7) * 8;
    const int j = 32 * half + jr;
    if (j < prev_n) {
      __hip_bfloat16* yr = p.y + (prev_row0 + j) * kD + cc;
#pragma unroll
      for (int i = 0; i < 8; ++i) yr[i] = __float2bfloat16(half == 0 ? ymine[i] + pv[i] : pv[i] + ymine[i]);
    }
  };

  for (int s = pair; s < p.streams && !failed; s += p.n_pairs) {
    const int64_t tok0 = (int64_t)s * p.N;
    // ---- this wave's state, AGPR-resident ----
    // W1m[ct]: rows c = 32ct + crow, cols h = hs + lr   (W1[h][c])
    // W2m[ct]: rows h = hs + crow, cols c = 32ct + lr   (W2[c][h])
    Tile W1m[2], S1m[2], W2m[2], S2m[2];
    float m1 = 0.f, m2 = 0.f;   // this lane's max |W|,|S| per layer (for the operand scales)
    {
      const float* Wi = p.W_in + (int64_t)s * kP;
      const float* Si = p.S_in + (int64_t)s * kP;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c1 = 32 * ct + crow(r, lg), h1 = hs + lr;
          const float w1 = Wi[h1 * kD + c1], s1 = Si[h1 * kD + c1];
          W1m[ct].r[r] = ag_put(w1);
          S1m[ct].r[r] = ag_put(s1);
          m1 = fmaxf(m1, fmaxf(fabsf(w1), fabsf(s1)));
          const int h2 = hs + crow(r, lg), c2 = 32 * ct + lr;
          const float w2 = Wi[kH * kD + c2 * kH + h2], s2 = Si[kH * kD + c2 * kH + h2];
          W2m[ct].r[r] = ag_put(w2);
          S2m[ct].r[r] = ag_put(s2);
          m2 = fmaxf(m2, fmaxf(fabsf(w2), fabsf(s2)));
        }
    }

    for (int c0 = 0; c0 < p.N; c0 += p.chunk) {
      const int n = min(p.chunk, p.N - c0);

      // ================= the chunk's K, K^T, Q (fp16) and gates into LDS =================
      {
        // rows come from the staging area when the previous chunk prefetched them
        if (staged) __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's staging loads (long done)
        const ChunkRegs cr = staged ? unstage_chunk_regs(smem + OFF_STAGE, n, tid) : load_chunk_regs(p, tok0 + c0, gate_base(p, s, c0), n, tid);
        const int j = tid >> 2, cb = (tid & 3) * 16;
        _Float16 kv[16], qv[16];
        bf16x8_to_h(cr.k0, kv);
        bf16x8_to_h(cr.k1, kv + 8);
        bf16x8_to_h(cr.q0, qv);
        bf16x8_to_h(cr.q1, qv + 8);
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          *(h4*)(sK + j * RS + cb + i) = h4{kv[i], kv[i + 1], kv[i + 2], kv[i + 3]};
          *(h4*)(sQ + j * RS + cb + i) = h4{qv[i], qv[i + 1], qv[i + 2], qv[i + 3]};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sKT[(cb + i) * RS + j] = kv[i];
        if (tid < kB) {
          cf[COEF_THETA + tid] = cr.gt;
          float2* pairs = (float2*)(smem + OFF_COEF + COEF_PAIR);
          pairs[tid] = make_float2(1.f - cr.ga, cr.ge);
        }
        if (tid < 2) ci[tid] = 0;
      }
      {
        const float wm2 = wave_max(m2);
        if (lane == 0) ci[INT_M2 + w] = __float_as_int(wm2);
      }
      __syncthreads();
      // the next chunk's rows go straight to the staging area (read at its start)
      int next_s = s, next_c0 = c0 + p.chunk;
      if (next_c0 >= p.N) { next_s = s + p.n_pairs; next_c0 = 0; }
      const bool has_next = next_s < p.streams && p.N > 0;
      if (has_next)
        prefetch_chunk_lds(p, (int64_t)next_s * p.N + next_c0, gate_base(p, next_s, next_c0), min(p.chunk, p.N - next_c0),
                           tid, smem + OFF_STAGE);
      staged = has_next;

      // state scales: W1/S1 per wave; W2/S2 joint over the workgroup (the
      // half's O is one contraction over all its waves' W2 copies)
      const int e1 = scale_exp(wave_max(m1));
      const int e2 = scale_exp(fmaxf(fmaxf(__int_as_float(ci[INT_M2]), __int_as_float(ci[INT_M2 + 1])),
                                     fmaxf(__int_as_float(ci[INT_M2 + 2]), __int_as_float(ci[INT_M2 + 3]))));
      const float f1 = pow2pos(e1), f2 = pow2pos(e2);

      // ================= a2: key-side forward Z1 = K W1^T (rows j, cols h) =================
      // A1 = SiLU(Z1) (scaled fp16: kept for the update, copied to LDS for the
      // contractions over h), SiLU'(Z1) (fp16, for backprop)
      h8 A1h[2][2], SPh[2][2];
      h8 w1f[2][2];   // W1 operand fragments (scaled fp16), reused by the layer-1 retrieval
      int eA1;
      {
        f16v Z[2];
        float am = 0.f;
        f16v zacc[2] = {{}, {}};
        const float zun = pow2neg(e1);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            w1f[ct][st] = state_frag(W1m[ct], st, f1);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
              zacc[jt] = mfma(lds_frag(sK + (32 * jt + lr) * RS, 32 * ct + 16 * st, lg), w1f[ct][st], zacc[jt]);
          }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          const f16v acc = zacc[jt];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float z = acc[r] * zun;
            const float sg = sigmoidf_(z);
            const float a = z * sg;
            Z[jt][r] = a;
            am = fmaxf(am, fabsf(a));
            SPh[jt][r >> 3][r & 7] = (_Float16)(sg + a * (1.f - sg));   // s (1 + z (1 - s))
          }
        }
        {
          const float wam = wave_max(am);
          if (lane == 0) ci[INT_MA1 + w] = __float_as_int(wam);
        }
        // W2 fragments (workgroup-wide scale) and this wave's two W2 copies:
        // [h_l][c] for the backprop, [c][h_l] for the half's O (the fragment
        // slots follow the operand order 16s + 8(i/4) + 4lg + i%4 over h_l)
        h8 w2f[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            w2f[ct][st] = state_frag(W2m[ct], st, f2);
            _Float16* row = sRW2 + (32 * ct + lr) * RSA + 16 * st + 4 * lg;
            *(h4*)row = h4{w2f[ct][st][0], w2f[ct][st][1], w2f[ct][st][2], w2f[ct][st][3]};
            *(h4*)(row + 8) = h4{w2f[ct][st][4], w2f[ct][st][5], w2f[ct][st][6], w2f[ct][st][7]};
          }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sRW[crow(r, lg) * RS + 32 * ct + lr] = w2f[ct][r >> 3][r & 7];
        __syncthreads();   // every wave's A1 maximum and W2 copies
        // A1 with the workgroup-wide scale, kept for the update and copied to LDS
        eA1 = scale_exp(fmaxf(fmaxf(__int_as_float(ci[INT_MA1]), __int_as_float(ci[INT_MA1 + 1])),
                              fmaxf(__int_as_float(ci[INT_MA1 + 2]), __int_as_float(ci[INT_MA1 + 3]))));
        const float fA1 = pow2pos(eA1);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const _Float16 hv = (_Float16)(Z[jt][r] * fA1);
            A1h[jt][r >> 3][r & 7] = hv;
            sRA[(32 * jt + crow(r, lg)) * RSA + lr] = hv;   // A1 copy [j][h_l]
          }
      }
      __syncthreads();   // every wave's A1 copy

      // ================= this half's O^T = W2 A1^T over its 128 hidden units =================
      // wave w: the 32 x 32 tile (tokens 32 jt.., columns 32 ct..), jt = w >> 1,
      // ct = w & 1, straight from the four waves' A1 and W2 [c][h_l] copies;
      // lane = token j = 32 jt + lr, its 16 columns c = 32 ct + 8g + 4lg + q
      // (register 4g + q)
      float om[16];
      const int tj = 32 * (w >> 1) + lr, tc = 32 * (w & 1) + 4 * lg;
      {
        f16v acc = {};
#pragma unroll
        for (int src = 0; src < kWaves; ++src) {
          const _Float16* a1 = (const _Float16*)(smem + OFF_WAVE + src * kWaveRegion);
          const _Float16* w2 = (const _Float16*)(smem + OFF_WAVE + src * kWaveRegion + kA1Bytes + kW2Bytes);
#pragma unroll
          for (int st = 0; st < 2; ++st)
            acc = mfma(lds_frag(w2 + (32 * (w & 1) + lr) * RSA, 16 * st, lg),
                       lds_frag(a1 + (32 * (w >> 1) + lr) * RSA, 16 * st, lg), acc);
        }
        const float co = pow2neg(eA1 + e2);
#pragma unroll
        for (int r = 0; r < 16; ++r) om[r] = acc[r] * co;
      }
      // publish this half's O (and, implied by the flag, last chunk's y partial)
      const unsigned par = seq & 1u;
#pragma unroll
      for (int e = 0; e < 8; ++e) xstore2(xO_me + par * kB * kD, e, tid, om[2 * e], om[2 * e + 1]);

      // loads issued right after this half's flag: this chunk's V (used
      // after the handshake)
      uint2 vq[4] = {make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0)};
      auto issue_loads = [&] {
        // V[tj][tc + 8g .. +3] for this thread's O elements
        if (tj < n) {
#pragma unroll
          for (int g = 0; g < 4; ++g) vq[g] = *(const uint2*)(p.v + (tok0 + c0 + tj) * kD + tc + 8 * g);
        }
      };

      // ================= a1: coefficients (both halves compute them identically) =================
      // Run by waves 1..3 while thread 0 of wave 0 awaits the partner (first
      // used after that barrier).  Lane m of each wave holds token m's
      // (1 - alpha_m, eta_m).
      //
      // D, one lane per column i: t = theta_i prod_{i<m<=j} eta_m, started at
      // j == i by adding theta_i to a zero product, and
      // D[j][i] = (1 - alpha_j) D[j-1][i] + t -- one fma per row on each of the
      // two carried values, the row's gates broadcast with readlane.  Wave 3
      // runs rows 0..31 and wave 1 rows 32..63.  For columns i >= 32 wave 1's
      // rows are exact (their recurrences start at row i); for i < 32 wave 1
      // starts from zero, and the rows are completed after the wait from wave
      // 3's carried pair at row 31 through the (column-independent) transfer
      //   (D, t)_j = (T11_j D_31 + T12_j t_31, T22_j t_31),
      // T11_j = prod_{32<=m<=j} (1 - alpha_m), T22_j = prod_{32<=m<=j} eta_m,
      // T12_j = sum_{32<=l<=j} prod_{l<m<=j} (1 - alpha_m) T22_l,
      // which wave 2 gets from prefix scans restarted at row 32.
      auto coef_work = [&] {
      if (w >= 1) {
        const float2 gl = ((const float2*)(smem + OFF_COEF + COEF_PAIR))[lane];
        if (w != 2) {
          const int i = lane;
          const int j0 = __builtin_amdgcn_readfirstlane(w == 3 ? 0 : 32);
          const float thi = cf[COEF_THETA + i];
          float di = 0.f, t = 0.f;
          float* drow = sDM + j0 * RSF + i;
          // the 32 rows stay in registers and are stored after the loop, so the
          // gate reads below never wait behind row stores
          float drows[32];
          auto step = [&](int jj, float ga, float ge) {
            // theta_i in lane j only: a select on the lane mask 1 << j
            float inj;
            asm("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(inj) : "v"(thi), "s"(1ull << (j0 + jj)));
            t = fmaf(ge, t, inj);
            di = fmaf(ga, di, t);
            drows[jj] = di;
          };
          // the steps' (1 - alpha_j, eta_j) pairs (padding included) as LDS
          // broadcasts, two steps per 16-byte read, 16 steps per batch
          const float4* pairs4 = (const float4*)(smem + OFF_COEF + COEF_PAIR) + j0 / 2;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float4 g[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) g[q] = pairs4[8 * b + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              step(16 * b + 2 * q, g[q].x, g[q].y);
              step(16 * b + 2 * q + 1, g[q].z, g[q].w);
            }
          }
#pragma unroll
          for (int jj = 0; jj < 32; ++jj) drow[jj * RSF] = drows[jj];
          // wave 3: t at row 31 for i < 32; wave 1: t at row 63 (= U_i) for i >= 32
          if ((w == 3) == (i < 32)) cf[COEF_XT + i] = t;
        } else {
          // lane j = token j: E_j by a prefix product of eta, then (A_j, F_j) by
          // a prefix scan of the maps u -> (1 - alpha_j) u + E_j (A_j is the
          // scan's product part, F_j its value from F_{-1} = 0)
          const float e = wave_prefix_prod(gl.y);
          float a = gl.x, f = e;
          wave_affine_scan(a, f);
          cf[COEF_A + lane] = a;
          cf[COEF_E + lane] = e;
          cf[COEF_F + lane] = f;
          // the same scans restarted at row 32 (identity maps below it)
          const bool lo = lane < 32;
          const float e2 = wave_prefix_prod(lo ? 1.f : gl.y);
          float a2 = lo ? 1.f : gl.x, f2 = lo ? 0.f : e2;
          wave_affine_scan(a2, f2);
          if (!lo) {
            cf[COEF_T11 + lane - 32] = a2;
            cf[COEF_T12 + lane - 32] = f2;
          }
          if (lane == 63) ci[INT_T22] = __float_as_int(e2);
        }
      }
      };

      if (!handshake(seq + 2, issue_loads, coef_work)) { failed = true; break; }
      // the partner's data (published before its flag) is loaded now and
      // used after the D completion, the update weights and SC1
      float pvv[16], pyv[8];
      xload8(xO_pt + par * kB * kD, 0, tid, pvv);       // the partner's values of this thread's O elements
      xload8(xO_pt + par * kB * kD, 4, tid, pvv + 8);
      if (prev_row0 >= 0) load_prev_y(par ^ 1u, pyv);
      {
        // D rows 32..63 of columns 0..31: 8 row groups x 32 columns, 4 rows each
        const int i = tid & 31, jr = 32 + 4 * (tid >> 5);
        const float d31 = sDM[31 * RSF + i], t31 = cf[COEF_XT + i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sDM[(jr + q) * RSF + i] = fmaf(cf[COEF_T11 + jr + q - 32], d31, cf[COEF_T12 + jr + q - 32] * t31);
      }
      __syncthreads();
      if (w == 3) {
        // weights of the state update: U_i = theta_i prod_{m>i} eta_m and
        // D[n-1][i], each scaled into (0.5, 1] for fp16 (padding has eta = 1)
        const int i = lane;
        const float ti = cf[COEF_XT + i];
        const float ui = i < 32 ? ti * __int_as_float(ci[INT_T22]) : ti;
        const float dlast = sDM[(n - 1) * RSF + i];
        const float mu = wave_max(fabsf(ui)), md = wave_max(fabsf(dlast));
        int eu = 0, ed = 0;
        if (mu > 0.f && mu < INFINITY) { (void)frexpf(mu, &eu); eu = -eu; }
        if (md > 0.f && md < INFINITY) { (void)frexpf(md, &ed); ed = -ed; }
        ch[H16_WU + i] = (_Float16)ldexpf(ui, eu);
        ch[H16_WD + i] = (_Float16)ldexpf(dlast, ed);
        if (lane == 0) { ci[INT_EWU] = eu; ci[INT_EWD] = ed; }
      }

      // last chunk's y rows (the partner published them before this flag)
      if (prev_row0 >= 0) finish_prev_y(pyv);

      // ================= first-layer scores SC1 = D o (Q K^T): one 32x32 tile per wave =================
      f16v sc;
      if constexpr (kRW) {
        const int jt = w >> 1, it = w & 1;
        f16v acc = {};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int st = 0; st < 2; ++st)
            acc = mfma(lds_frag(sQ + (32 * jt + lr) * RS, 32 * ct + 16 * st, lg),
                       lds_frag(sK + (32 * it + lr) * RS, 32 * ct + 16 * st, lg), acc);
        float am = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = acc[r] * sDM[(32 * jt + crow(r, lg)) * RSF + 32 * it + lr];
          am = fmaxf(am, fabsf(sc[r]));
        }
        am = wave_max(am);
        if (lane == 0) atomicMax((unsigned int*)&ci[INT_AMAX_SC1], __float_as_uint(am));
      }

      // ================= O = half 0 + half 1, Delta2 = O - V =================
      float d2v[16];
      {
        float am = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const unsigned vw[2] = {vq[g].x, vq[g].y};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * g + q;
            const float o = half == 0 ? om[r] + pvv[r] : pvv[r] + om[r];
            const float vv = __uint_as_float((q & 1) ? (vw[q >> 1] & 0xffff0000u) : (vw[q >> 1] << 16));
            d2v[r] = tj < n ? o - vv : 0.f;
            am = fmaxf(am, fabsf(d2v[r]));
          }
        }
        am = wave_max(am);
        if (lane == 0) atomicMax((unsigned int*)&ci[INT_AMAX_D2], __float_as_uint(am));
      }
      __syncthreads();   // every wave's SC1 and Delta2 amax is in
      const int eSC = scale_exp(__uint_as_float((unsigned)ci[INT_AMAX_SC1]));
      const float fSC = pow2pos(eSC);
      if constexpr (kRW) {
        const int jt = w >> 1, it = w & 1;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sSC1[(32 * jt + crow(r, lg)) * RS + 32 * it + lr] = (_Float16)(sc[r] * fSC);
      }
      const int eD2 = scale_exp(__uint_as_float((unsigned)ci[INT_AMAX_D2]));
      const float fD2 = pow2pos(eD2);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        h4 hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = (_Float16)(d2v[4 * g + q] * fD2);
          sD2T[(tc + 8 * g + q) * RS + tj] = hv[q];
        }
        *(h4*)(sD2 + tj * RS + tc + 8 * g) = hv;
      }
      __syncthreads();

      // ================= a3: Delta1 = (Delta2 W2) * SiLU'(Z1)  (rows j, cols h) =================
      h8 D1h[2][2];
      int eD1;
      {
        f16v Df[2];
        float am = 0.f;
        const float dun = pow2neg(eD2 + e2);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f16v acc = {};
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int st = 0; st < 2; ++st)
              acc = mfma(lds_frag(sD2 + (32 * jt + lr) * RS, 32 * ct + 16 * st, lg),
                         lds_frag(sRW + lr * RS, 32 * ct + 16 * st, lg), acc);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = acc[r] * dun * (float)SPh[jt][r >> 3][r & 7];
            Df[jt][r] = x;
            am = fmaxf(am, fabsf(x));
          }
        }
        eD1 = scale_exp(wave_max(am));
        const float fD1 = pow2pos(eD1);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) D1h[jt][r >> 3][r & 7] = (_Float16)(Df[jt][r] * fD1);
      }

      // ================= a5 layer 1: Zq1^T = W1 (A q)^T + S1 (F q)^T - Delta1^T SC1^T (rows h, cols j) =================
      // One accumulator per token tile: the query fragment of token j (lane
      // column) is scaled by A_j 2^s_j for the W1 product and by F_j 2^s_j for
      // the S1 product; W1 and S1 fragments are converted once for both tiles.
      h8 H1h[2][2];
      int eH1[2];
      if constexpr (kRW) {
        _Float16 ajh[2], fjh[2];
        int sj[2];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          token_factors(cf[COEF_A + 32 * jt + lr], cf[COEF_F + 32 * jt + lr], ajh[jt], fjh[jt], sj[jt]);
        f16v accZ[2] = {};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 wf = w1f[ct][st], sf = state_frag(S1m[ct], st, f1);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const h8 qf = lds_frag(sQ + (32 * jt + lr) * RS, 32 * ct + 16 * st, lg);
              accZ[jt] = mfma(wf, hscale(qf, ajh[jt]), accZ[jt]);
              accZ[jt] = mfma(sf, hscale(qf, fjh[jt]), accZ[jt]);
            }
          }
        const float c3 = pow2neg(eD1 + eSC);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f16v acc3 = {};
#pragma unroll
          for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int st = 0; st < 2; ++st)
              acc3 = mfma(D1h[it][st], lds_frag(sSC1 + (32 * jt + lr) * RS, 32 * it + 16 * st, lg), acc3);
          const float cz = pow2neg(e1 + sj[jt]);
          f16v Hf;
          float am = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float z = fmaf(acc3[r], -c3, accZ[jt][r] * cz);
            Hf[r] = z * sigmoidf_(z);
            am = fmaxf(am, fabsf(Hf[r]));
          }
          eH1[jt] = scale_exp(wave_max(am));
          const float fH = pow2pos(eH1[jt]);
#pragma unroll
          for (int r = 0; r < 16; ++r) H1h[jt][r >> 3][r & 7] = (_Float16)(Hf[r] * fH);
        }
      }
      else {
        // chunk-start read: Zq1^T = W1_0 q^T
        f16v accZ[2] = {};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 wf = w1f[ct][st];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
              accZ[jt] = mfma(wf, lds_frag(sQ + (32 * jt + lr) * RS, 32 * ct + 16 * st, lg), accZ[jt]);
          }
        const float cz = pow2neg(e1);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f16v Hf;
          float am = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float z = accZ[jt][r] * cz;
            Hf[r] = z * sigmoidf_(z);
            am = fmaxf(am, fabsf(Hf[r]));
          }
          eH1[jt] = scale_exp(wave_max(am));
          const float fH = pow2pos(eH1[jt]);
#pragma unroll
          for (int r = 0; r < 16; ++r) H1h[jt][r >> 3][r & 7] = (_Float16)(Hf[r] * fH);
        }
      }

      const float An = cf[COEF_A + n - 1], En = cf[COEF_E + n - 1], Fn = cf[COEF_F + n - 1];
      const int ewU = ci[INT_EWU], ewD = ci[INT_EWD];
      float m1n = 0.f, m2n = 0.f;
      const float uD1 = pow2neg(ewD + eD1), uU1 = pow2neg(ewU + eD1);
      const float uD2 = pow2neg(ewD + eA1 + eD2), uU2 = pow2neg(ewU + eA1 + eD2);
      // ================= a4, layer 1 (W1, S1 are not read again this chunk) =================
      // G1^T[c][h] = sum_j K[j][c] w_j Delta1[j][h]
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f16v gU = {}, gD = {};
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 kf = lds_frag(sKT + (32 * ct + lr) * RS, 32 * jt + 16 * st, lg);
            gU = mfma(hmul(kf, lds_frag(ch + H16_WU, 32 * jt + 16 * st, lg)), D1h[jt][st], gU);
            gD = mfma(hmul(kf, lds_frag(ch + H16_WD, 32 * jt + 16 * st, lg)), D1h[jt][st], gD);
          }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float w0 = ag_get(W1m[ct].r[r]), s0 = ag_get(S1m[ct].r[r]);
          const float wn = An * w0 + Fn * s0 - gD[r] * uD1;
          const float sn = En * s0 - gU[r] * uU1;
          W1m[ct].r[r] = ag_put(wn);
          S1m[ct].r[r] = ag_put(sn);
          m1n = fmaxf(m1n, fmaxf(fabsf(wn), fabsf(sn)));
        }
      }

      // ================= masked second-layer scores (D o (H1 A1^T))^T (rows i, cols j) =================
      h8 DPh[2][2][2];
      int eDP[2];
      if constexpr (kRW)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        f16v Pf[2];
        float am = 0.f;
        const int j = 32 * jt + lr;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          f16v acc = {};
#pragma unroll
          for (int st = 0; st < 2; ++st)
            acc = mfma(lds_frag(sRA + (32 * it + lr) * RSA, 16 * st, lg), H1h[jt][st], acc);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f4v dv = *(const f4v*)(sDM + j * RSF + 32 * it + 8 * g + 4 * lg);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // unscaled by 2^-(eA1 + eH1) through the exponent below, not per element
              const float x = acc[4 * g + q] * dv[q];
              Pf[it][4 * g + q] = x;
              am = fmaxf(am, fabsf(x));
            }
          }
        }
        const int er = scale_exp(wave_max(am));
        const float fr = pow2pos(er);
        eDP[jt] = er + eA1 + eH1[jt];   // the scale of the true scores
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int r = 0; r < 16; ++r) DPh[it][jt][r >> 3][r & 7] = (_Float16)(Pf[it][r] * fr);
      }

      // ================= a5 layer 2: y^T partial = W2 (A H1)^T + S2 (F H1)^T - Delta2^T (D o P)^T =================
      // tiles go straight to this wave's region (fp32 [c][j]): the wave is past
      // its last read of its A1 and W2 copies, and other waves read the region
      // only after the next barrier.  As in layer 1, one accumulator per tile
      // with the per-token factors on the H1 fragments.
      if constexpr (kRW) {
        _Float16 ajh[2], fjh[2];
        int sj[2];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          token_factors(cf[COEF_A + 32 * jt + lr], cf[COEF_F + 32 * jt + lr], ajh[jt], fjh[jt], sj[jt]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f16v accY[2] = {};
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 wf = state_frag(W2m[ct], st, f2), sf = state_frag(S2m[ct], st, f2);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              accY[jt] = mfma(wf, hscale(H1h[jt][st], ajh[jt]), accY[jt]);
              accY[jt] = mfma(sf, hscale(H1h[jt][st], fjh[jt]), accY[jt]);
            }
          }
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            f16v acc3 = {};
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
              for (int st = 0; st < 2; ++st)
                acc3 = mfma(lds_frag(sD2T + (32 * ct + lr) * RS, 32 * it + 16 * st, lg), DPh[it][jt][st], acc3);
            const float cy = pow2neg(e2 + eH1[jt] + sj[jt]), c3 = pow2neg(eD2 + eDP[jt]);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {   // rows c = 32ct + 8g4 + 4lg + 0..3 are consecutive
              f4v o;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int r = 4 * g4 + q;
                o[q] = fmaf(acc3[r], -c3, accY[jt][r] * cy);
              }
              *(f4v*)(sRF + (32 * jt + lr) * RSF + 32 * ct + 8 * g4 + 4 * lg) = o;
            }
          }
        }
      }
      else {
        // chunk-start read: y^T partial = W2_0 H1^T
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          f16v accY[2] = {};
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 wf = state_frag(W2m[ct], st, f2);
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) accY[jt] = mfma(wf, H1h[jt][st], accY[jt]);
          }
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const float cy = pow2neg(e2 + eH1[jt]);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              f4v o;
#pragma unroll
              for (int q = 0; q < 4; ++q) o[q] = accY[jt][4 * g4 + q] * cy;
              *(f4v*)(sRF + (32 * jt + lr) * RSF + 32 * ct + 8 * g4 + 4 * lg) = o;
            }
          }
        }
      }

      // ================= a4, layer 2: G2^T[h][c] = sum_j A1[j][h] w_j Delta2[j][c] =================
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f16v gU = {}, gD = {};
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const h8 df = lds_frag(sD2T + (32 * ct + lr) * RS, 32 * jt + 16 * st, lg);
            gU = mfma(A1h[jt][st], hmul(df, lds_frag(ch + H16_WU, 32 * jt + 16 * st, lg)), gU);
            gD = mfma(A1h[jt][st], hmul(df, lds_frag(ch + H16_WD, 32 * jt + 16 * st, lg)), gD);
          }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float w0 = ag_get(W2m[ct].r[r]), s0 = ag_get(S2m[ct].r[r]);
          const float wn = An * w0 + Fn * s0 - gD[r] * uD2;
          const float sn = En * s0 - gU[r] * uU2;
          W2m[ct].r[r] = ag_put(wn);
          S2m[ct].r[r] = ag_put(sn);
          m2n = fmaxf(m2n, fmaxf(fabsf(wn), fabsf(sn)));
        }
      }
      __syncthreads();

      // ---- this half's y: sum the 4 wave partials; send the partner its rows, keep mine ----
      {
        const int jr = tid >> 3, cc = (tid & 7) * 8;
        float send[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { send[i] = 0.f; ymine[i] = 0.f; }
#pragma unroll
        for (int src = 0; src < kWaves; ++src) {
          const float* rp = (const float*)(smem + OFF_WAVE + src * kWaveRegion);
          const float* ps = rp + (32 * (1 - half) + jr) * RSF + cc;
          const float* pm = rp + (32 * half + jr) * RSF + cc;
          const f4v s0 = *(const f4v*)ps, s1 = *(const f4v*)(ps + 4);
          const f4v m0 = *(const f4v*)pm, m1v = *(const f4v*)(pm + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            send[i] += s0[i]; send[4 + i] += s1[i];
            ymine[i] += m0[i]; ymine[4 + i] += m1v[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 8; i += 2) xstore2(xY_me + par * 32 * kD, i / 2, tid, send[i], send[i + 1]);
      }
      m1 = m1n;
      m2 = m2n;
      prev_row0 = tok0 + c0;
      prev_n = n;
      ++seq;
      __syncthreads();   // LDS tiles and wave regions are rewritten by the next chunk
    }

    if (failed) {
      // partner never arrived: poison this stream's state so the failure is visible
      float* Wo = p.W_out + (int64_t)s * kP;
      float* So = p.S_out + (int64_t)s * kP;
      for (int i = tid; i < kP; i += kThreads) { Wo[i] = __builtin_nanf(""); So[i] = __builtin_nanf(""); }
      break;
    }
    // ---- write this wave's part of the final state ----
    {
      float* Wo = p.W_out + (int64_t)s * kP;
      float* So = p.S_out + (int64_t)s * kP;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c1 = 32 * ct + crow(r, lg), h1 = hs + lr;
          Wo[h1 * kD + c1] = ag_get(W1m[ct].r[r]);
          So[h1 * kD + c1] = ag_get(S1m[ct].r[r]);
          const int h2 = hs + crow(r, lg), c2 = 32 * ct + lr;
          Wo[kH * kD + c2 * kH + h2] = ag_get(W2m[ct].r[r]);
          So[kH * kD + c2 * kH + h2] = ag_get(S2m[ct].r[r]);
        }
    }
  }

  // the last chunk's y rows: one more handshake (a flag value no chunk uses)
  if (!failed && prev_row0 >= 0) {
    if (handshake(seq + 2, nothing, nothing)) {
      float pyv[8];
      load_prev_y((seq - 1) & 1u, pyv);
      finish_prev_y(pyv);
    }
  }
  // no load into this workgroup's LDS may outlive it (a pair that gave up
  // can leave a staging prefetch in flight)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace

bool mlp2_supported(const Shape& s, int chunk) {
  return s.L == 2 && s.d == kD && s.hidden == kH && s.io == TM_IO_BF16 &&
         (s.read_mode == TM_READ_AFTER_WRITE || s.read_mode == TM_READ_CHUNK_START) && chunk >= 1 && chunk <= kB;
}

static int64_t pairs_for(const Shape& s) { return s.streams < kMaxPairs ? s.streams : kMaxPairs; }

int64_t mlp2_ws_bytes(const Shape& s, int) {
  const int64_t np = pairs_for(s);
  return np * kPairBytes + 2 * np * kFlagStride + 256;
}

hipError_t launch_mlp2(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                       const float* alpha, const float* eta, const float* theta,
                       const float* W_in, const float* S_in, void* y, float* W_out,
                       float* S_out, void* ws, hipStream_t stream) {
  // the kernel's dynamic LDS size, set on every call (no state kept between
  // calls; idempotent and cheap next to the kernel)
  const void* kfn = s.read_mode == TM_READ_AFTER_WRITE ? (const void*)mlp2_pair_kernel<true>
                                                       : (const void*)mlp2_pair_kernel<false>;
  hipError_t e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // every pair must be resident at once (one workgroup per CU)
  int64_t np = pairs_for(s);
  if (np > cus / 2) np = cus / 2;
  if (np < 1) return hipErrorInvalidConfiguration;
  Params p;
  p.N = s.N;
  p.chunk = chunk;
  p.streams = s.streams;
  p.n_pairs = (int)np;
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
  p.flags = (unsigned*)(base + pairs_for(s) * kPairBytes);
  p.status = (unsigned*)(base + pairs_for(s) * kPairBytes + 2 * pairs_for(s) * kFlagStride);
  p.spin_max = kSpinMax;
  p.chunk_gates = s.chunk_gates;
  hipLaunchKernelGGL(zero_flags_kernel, dim3(1), dim3(256), 0, stream, p.flags, (int)(2 * np), p.status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.read_mode == TM_READ_AFTER_WRITE)
    hipLaunchKernelGGL(mlp2_pair_kernel<true>, dim3((unsigned)(2 * np)), dim3(kThreads), kLdsBytes, stream, p);
  else
    hipLaunchKernelGGL(mlp2_pair_kernel<false>, dim3((unsigned)(2 * np)), dim3(kThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace titans
