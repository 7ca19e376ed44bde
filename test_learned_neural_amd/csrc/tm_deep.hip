// Deep-memory path on the matrix cores: bias-free SiLU MLP memories of any
// depth L >= 2 whose widths are multiples of 64, bf16 io, chunk <= 256.
//
// The method is the chunked form of "Titans: Learning to Memorize at Test
// Time" (mer.dev notes, section 3.2: every gradient of a chunk is taken at
// the chunk-start weights W_0), evaluated per chunk in closed form:
//
//   coefficients  A_j = prod_{m<=j}(1 - alpha_m), E_j = prod_{m<=j} eta_m,
//                 F_j = (1 - alpha_j) F_{j-1} + E_j, U_i = theta_i prod_{m>i} eta_m,
//                 D[j,i] = (1 - alpha_j) D[j-1,i] + theta_i prod_{i<m<=j} eta_m, D[i,i] = theta_i
//                 (the section 3.1 update rules unrolled over the chunk)
//   key side      z^l = a^{l-1} W_0^l^T, a^l = SiLU(z^l), delta^L = a^L - V,
//                 delta^{l-1} = (delta^l W_0^l) * SiLU'(z^{l-1})
//   fold          W^l <- A_n W^l + F_n S^l - sum_j D[n-1,j] delta^l_j a^{l-1}_j^T
//                 S^l <- E_n S^l - sum_j U_j delta^l_j a^{l-1}_j^T
//   retrieval     zq^l = diag(A) h W_0^l^T + diag(F) h S_0^l^T - (D o (h a^{l-1 T})) delta^l,
//                 h <- SiLU(zq^l), y = zq^L  (section 3.1 "Retrieving a Memory": the
//                 state after each token's write, with no weight change)
//
// Mapping on gfx950.  A deep memory's state (5.2 MB per stream at d = 128,
// hidden 512, four layers, W and S in fp32) fits neither one CU nor a few, so
// every step of a chunk is one launch over all streams, its output tiles
// (64 x 64, four waves each holding a 32 x 32 block) spread over the CUs:
//
//   sweep (caller's stream)  key(1) .. key(L), back(L) .. back(2), fold
//   reads (a second stream)  scores(1), read(1), .. scores(L), read(L)
//
// The reads of chunk c need the chunk-start state and the chunk's
// activations and deltas, not the fold, so they run beside the fold of
// chunk c and the sweep of chunk c + 1.  Every contraction runs on
// v_mfma_f32_32x32x16_bf16 with bf16 operands and fp32 sums: both operands
// are staged through LDS in 64-deep k slices, the next slice's loads in
// flight during the current slice's products.  The operands always have k
// contiguous in memory; the producers write a transposed copy where a later
// contraction runs over the other index (the tokens of a^l and delta^l, the
// output units of W^l).
//
// The state stays fp32 in W_out / S_out, read and written only by the fold;
// the fold also leaves bf16 copies of the new state (W, S and W^T per layer)
// for the next chunk's products.  The copies rotate through three slots and
// the chunk intermediates through two regions of the workspace, so the
// reads of chunk c (slot c % 3, region c % 2) never meet the writes of the
// two chunks after it.  The fold's weights (D's last row, U) scale the
// deltas as they are staged.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

#include <mutex>

namespace titans {
namespace {

constexpr int kT = 64;                 // output tile rows and columns
constexpr int kThreads = 256;          // four waves
constexpr int kMaxChunkDeep = 256;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// Byte offsets in one stream's workspace (every array fp32).
struct DLayout {
  int b;   // token rows per region (the chunk rounded up to 64)
  int64_t act[kMaxLayers + 1];    // a^l [b][w_l], l = 1..L-1
  int64_t actT[kMaxLayers + 1];   // a^l transposed [w_l][b], l = 0..L-1 (a^0 = K)
  int64_t sp[kMaxLayers + 1];     // SiLU'(z^l) [b][w_l], l = 1..L-1
  int64_t dlt[kMaxLayers + 1];    // delta^l [b][w_l], l = 2..L
  int64_t dltT[kMaxLayers + 1];   // delta^l transposed [w_l][b], l = 1..L
  int64_t hq[2];                  // query-side activations [b][maxw], ping-pong
  int64_t P;                      // masked scores [b][b]
  int64_t D;                      // decay weights [b][b]
  int64_t coef;                   // A, E, F, U, D[n-1, :]: [5][b]
  int64_t region;                 // bytes per region
  int64_t copy;                   // bytes per state array (P floats, 256-byte aligned)
  int64_t slot;                   // bytes per slot: W, S and W^T (per layer [n_in][n_out])
  int64_t total;                  // bytes per stream: two regions and three slots
};

int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

DLayout deep_layout(const Shape& s, int chunk) {
  DLayout y{};
  const int rows = chunk < s.N ? chunk : (s.N > 0 ? s.N : 1);
  y.b = (rows + kT - 1) / kT * kT;
  const int64_t b = y.b;
  int64_t cur = 0;
  auto take = [&](int64_t floats) {
    const int64_t at = cur;
    cur += al256(floats * 4);
    return at;
  };
  for (int l = 1; l < s.L; ++l) y.act[l] = take(b * s.widths[l]);
  for (int l = 0; l < s.L; ++l) y.actT[l] = take(b * s.widths[l]);
  for (int l = 1; l < s.L; ++l) y.sp[l] = take(b * s.widths[l]);
  for (int l = 2; l <= s.L; ++l) y.dlt[l] = take(b * s.widths[l]);
  for (int l = 1; l <= s.L; ++l) y.dltT[l] = take(b * s.widths[l]);
  y.hq[0] = take(b * s.maxw);
  y.hq[1] = take(b * s.maxw);
  y.P = take(b * b);
  y.D = take(b * b);
  y.coef = take(5 * b);
  y.region = cur;
  y.copy = al256(s.P * 4);
  y.slot = 3 * y.copy;
  y.total = 2 * y.region + 3 * y.slot;
  return y;
}

struct DP {
  int N, d, L, chunk, nch, read_mode, chunk_gates;
  int w[kMaxLayers + 1];
  int64_t off[kMaxLayers + 1];
  int64_t P;
  int maxw;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  uint16_t* y;
  const float* W_in;
  const float* S_in;
  float* W;
  float* S;
  unsigned char* ws;
  int64_t ws_stride;
  DLayout lay;
};

// Per-launch view of one stream's chunk: region and slot pointers.
struct View {
  int n, c0;
  unsigned char* reg;                  // this chunk's region
  const float *W0, *S0, *WT0;          // chunk-start state (slot c % 3)
  float *W1, *S1, *WT1;                // the fold's result (slot (c + 1) % 3)
};

__device__ __forceinline__ View view(const DP& p, int s, int c) {
  View v;
  v.c0 = c * p.chunk;
  v.n = min(p.chunk, p.N - v.c0);
  unsigned char* base = p.ws + (int64_t)s * p.ws_stride;
  v.reg = base + (int64_t)(c & 1) * p.lay.region;
  unsigned char* sr = base + 2 * p.lay.region + (int64_t)(c % 3) * p.lay.slot;
  unsigned char* sw = base + 2 * p.lay.region + (int64_t)((c + 1) % 3) * p.lay.slot;
  v.W0 = (const float*)sr;
  v.S0 = (const float*)(sr + p.lay.copy);
  v.WT0 = (const float*)(sr + 2 * p.lay.copy);
  v.W1 = (float*)sw;
  v.S1 = (float*)(sw + p.lay.copy);
  v.WT1 = (float*)(sw + 2 * p.lay.copy);
  return v;
}

template <class T>
__device__ __forceinline__ T* at(unsigned char* reg, int64_t off) {
  return (T*)(reg + off);
}

__device__ __forceinline__ float bf2f(unsigned short h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ unsigned short f2bf(float x) {   // round to nearest even
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
__device__ __forceinline__ float logistic(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float silu(float z) { return z * logistic(z); }
__device__ __forceinline__ float silu_prime(float z) {
  const float s = logistic(z);
  return s * (1.0f + z * (1.0f - s));
}

// An operand: element (row, k) at p[row * ld + k], k contiguous, fp32 (F32)
// or bf16; rows at or past `rows` read row rows - 1 (an address in range) and
// count as zero, and so does every k >= K.  Every source is laid out so that
// a 64-deep slice never reads past its allocation (rows padded to a multiple
// of 64 in k, or K a multiple of 64).
struct Src {
  const void* p;
  int64_t ld;
  int rows;
};

// Split operands: an fp32 value x is staged as hi = bf16(x) and lo = bf16(x -
// hi) (x - hi is exact in fp32), and a product of two split operands is
// summed as hi*hi + hi*lo + lo*hi, each term on the matrix cores with fp32
// sums: about 2^-16 relative per product instead of bf16's 2^-8.  bf16
// inputs (keys and queries) are exact and stage only hi.  A staged slice is
// 64 rows x KS k; its LDS tiles have row stride KS + 8 bf16.
template <int KS>
__host__ __device__ constexpr int tile_elems() { return kT * (KS + 8); }

template <bool F32, int KS>
struct Stage;

template <int KS>
struct Stage<true, KS> {   // fp32 source: pieces of 4 floats
  static constexpr int kQ = KS / 4;                      // pieces per row
  static constexpr int kPer = kT * kQ / kThreads;        // pieces per thread
  static constexpr int kRSt = KS + 8;
  float4 r[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads, row = e / kQ, kq = (e % kQ) * 4;
      r[u] = *(const float4*)((const float*)a.p + (int64_t)min(r0 + row, a.rows - 1) * a.ld + k0 + kq);
    }
  }
  // stores NC copies (hi tile 2c, lo tile 2c + 1 from `base`), copy c scaled
  // per k by ks[c] when KSCALE
  template <int NC, bool KSCALE>
  __device__ __forceinline__ void store(uint16_t* base, int rows_left, int k_left, const float* ks0, const float* ks1,
                                        int k0) const {
    constexpr int TE = tile_elems<KS>();
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads, row = e / kQ, kq = (e % kQ) * 4;
      const int kv = row < rows_left ? k_left - kq : 0;
      float x[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= kv) x[i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u16x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float xi = x[i];
          if constexpr (KSCALE) xi *= (c == 0 ? ks0 : ks1)[min(k0 + kq + i, kMaxChunkDeep - 1)];
          h[i] = f2bf(xi);
          l[i] = f2bf(xi - bf2f(h[i]));
        }
        *(u16x4*)(base + 2 * c * TE + row * kRSt + kq) = h;
        *(u16x4*)(base + (2 * c + 1) * TE + row * kRSt + kq) = l;
      }
    }
  }
};

template <int KS>
struct Stage<false, KS> {   // bf16 source: pieces of 8
  static constexpr int kQ = KS / 8;
  static constexpr int kPer = kT * kQ / kThreads;
  static constexpr int kRSt = KS + 8;
  uint4 r[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads, row = e / kQ, kq = (e % kQ) * 8;
      r[u] = *(const uint4*)((const uint16_t*)a.p + (int64_t)min(r0 + row, a.rows - 1) * a.ld + k0 + kq);
    }
  }
  template <int NC, bool KSCALE>
  __device__ __forceinline__ void store(uint16_t* base, int rows_left, int k_left, const float*, const float*,
                                        int) const {
    static_assert(NC == 1 && !KSCALE, "bf16 operands are staged once, unscaled");
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads, row = e / kQ, kq = (e % kQ) * 8;
      const int kv = row < rows_left ? k_left - kq : 0;
      u16x8 x = __builtin_bit_cast(u16x8, r[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= kv) x[i] = 0;
      *(u16x8*)(base + row * kRSt + kq) = x;
    }
  }
};

// acc[c][t] += A_c(m0 + i, k) B_t(n0 + j, k) summed over k < K, for the
// wave's 32 x 32 block (i, j in [0, 64)), as one pipeline: the next KS-deep
// slice's loads are in flight while the current slice is multiplied.  NA
// copies of A are staged from the same source, copy c with each element
// scaled by ks[c][k] (per-k weights in LDS) when KSCALE; NB operands B_t
// share the staged A.  LDS tiles: A copy c at hi 2c, lo 2c + 1, then B_t at
// hi 2 NA + 2t, lo 2 NA + 2t + 1.
// v_mfma_f32_32x32x16_bf16: lane l supplies row (A) or column (B) l % 32 with
// k values 8 (l / 32) .. + 7 of each 16-deep step; accumulator register r of
// lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
template <int KS, int NA, int NB, bool KSCALE, bool AF, bool BF>
__device__ void gemm(f32x16 (&acc)[NA][NB], const Src A, const Src (&B)[NB], int m0, int n0, int K,
                     const float* ks0, const float* ks1, uint16_t* lds) {
  constexpr int TE = tile_elems<KS>(), RS = KS + 8;
  uint16_t* const As = lds;
  uint16_t* const Bs = lds + 2 * NA * TE;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = (wv >> 1) * 32, wn = (wv & 1) * 32;
  Stage<AF, KS> sa;
  Stage<BF, KS> sb[NB];
  if (K <= 0) return;
  sa.fetch(A, m0, 0);
#pragma unroll
  for (int t = 0; t < NB; ++t) sb[t].fetch(B[t], n0, 0);
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int t = 0; t < NB; ++t)
      sb[t].template store<1, false>(Bs + 2 * t * TE, B[t].rows - n0, K - k0, nullptr, nullptr, k0);
    sa.template store<NA, KSCALE>(As, A.rows - m0, K - k0, ks0, ks1, k0);
    __syncthreads();
    if (k0 + KS < K) {
      sa.fetch(A, m0, k0 + KS);
#pragma unroll
      for (int t = 0; t < NB; ++t) sb[t].fetch(B[t], n0, k0 + KS);
    }
#pragma unroll
    for (int kk = 0; kk < KS; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const uint16_t* bt = Bs + 2 * t * TE + (wn + (lane & 31)) * RS + ko;
        const bf16x8 bh = *(const bf16x8*)bt;
        bf16x8 bl;
        if constexpr (BF) bl = *(const bf16x8*)(bt + TE);
#pragma unroll
        for (int c = 0; c < NA; ++c) {
          const uint16_t* ac = As + 2 * c * TE + (wm + (lane & 31)) * RS + ko;
          const bf16x8 ah = *(const bf16x8*)ac;
          acc[c][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[c][t], 0, 0, 0);
          if constexpr (BF) acc[c][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[c][t], 0, 0, 0);
          if constexpr (AF) {
            const bf16x8 al = *(const bf16x8*)(ac + TE);
            acc[c][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[c][t], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
}

// one A, one B
template <int KS, bool AF, bool BF>
__device__ __forceinline__ void gemm1(f32x16& acc, const Src A, const Src B, int m0, int n0, int K, uint16_t* lds) {
  f32x16 a[1][1] = {{acc}};
  const Src b[1] = {B};
  gemm<KS, 1, 1, false, AF, BF>(a, A, b, m0, n0, K, nullptr, nullptr, lds);
  acc = a[0][0];
}

// Row and column of accumulator register r in the tile at (m0, n0).
__device__ __forceinline__ int acc_row(int m0, int r) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  return m0 + (wv >> 1) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int n0) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  return n0 + (wv & 1) * 32 + (lane & 31);
}

// Stores the tile transposed: T[col][row .. row + 3] from registers 4g .. 4g + 3
// (four consecutive rows), one 16-byte store per group.
__device__ __forceinline__ void store_T(float* T, int64_t ldT, int m0, int n0, const float (&v)[16]) {
  const int col = acc_col(n0);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(float4*)(T + (int64_t)col * ldT + acc_row(m0, 4 * g)) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2],
                                                                           v[4 * g + 3]);
}

__device__ __forceinline__ const uint16_t* tok_rows(const uint16_t* base, const DP& p, int s, int c0) {
  return base + ((int64_t)s * p.N + c0) * p.d;
}

// the staging area every contraction of a kernel shares: six 64-deep tiles
// (hi and lo of two A copies and one B, or of one A and two B) or four
// 128-deep ones (hi and lo of one A and one B)
constexpr int kLdsElems = 6 * tile_elems<64>() > 4 * tile_elems<128>() ? 6 * tile_elems<64>() : 4 * tile_elems<128>();
__device__ __forceinline__ uint16_t* stage_lds() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[kLdsElems];
  return buf;
}

// ---- key side: z^l = a^{l-1} W_0^l^T (and, in layer 1's extra workgroup
// per stream, the chunk's coefficients and the transposed keys) ----
__global__ void __launch_bounds__(kThreads) deep_key_kernel(DP p, int c, int l) {
  const int s = blockIdx.y;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nout / kT, ntiles = ((n + kT - 1) / kT) * ntn;
  if ((int)blockIdx.x >= ntiles) {
    // coefficients of the chunk (one thread per column i of D; A, E, F on the last thread)
    __shared__ float gal[kMaxChunkDeep], get[kMaxChunkDeep], gth[kMaxChunkDeep];
    const int tid = threadIdx.x;
    const int64_t g0 = p.chunk_gates ? (int64_t)s * p.nch + c : (int64_t)s * p.N + v.c0;
    const int gs = p.chunk_gates ? 0 : 1;
    for (int j = tid; j < n; j += kThreads) {
      gal[j] = p.alpha[g0 + j * gs];
      get[j] = p.eta[g0 + j * gs];
      gth[j] = p.theta[g0 + j * gs];
    }
    __syncthreads();
    float* D = at<float>(v.reg, y.D);
    float* cf = at<float>(v.reg, y.coef);
    for (int i = tid; i < b; i += kThreads) {
      float di = 0.f, pr = 1.f;
      if (i < n) {
        const float ti = gth[i];
        di = ti;
        for (int j = 0; j < i; ++j) D[(int64_t)j * b + i] = 0.f;
        D[(int64_t)i * b + i] = di;
        for (int j = i + 1; j < n; ++j) {
          pr *= get[j];
          di = (1.f - gal[j]) * di + ti * pr;
          D[(int64_t)j * b + i] = di;
        }
        for (int j = n; j < b; ++j) D[(int64_t)j * b + i] = 0.f;
        cf[3 * b + i] = ti * pr;   // U
        cf[4 * b + i] = di;        // D[n-1, i]
      } else {
        for (int j = 0; j < b; ++j) D[(int64_t)j * b + i] = 0.f;
        cf[3 * b + i] = 0.f;
        cf[4 * b + i] = 0.f;
      }
    }
    if (tid == kThreads - 1) {
      float a = 1.f, e = 1.f, f = 0.f;
      for (int j = 0; j < n; ++j) {
        a *= 1.f - gal[j];
        e *= get[j];
        f = (1.f - gal[j]) * f + e;
        cf[j] = a;
        cf[b + j] = e;
        cf[2 * b + j] = f;
      }
    }
    // K^T [d][b] (fp32) for the fold's contraction over tokens
    const uint16_t* kr = tok_rows(p.k, p, s, v.c0);
    float* KT = at<float>(v.reg, y.actT[0]);
    for (int e = tid; e < n * (p.d / 8); e += kThreads) {
      const int j = e / (p.d / 8), c8 = (e % (p.d / 8)) * 8;
      const u16x8 x = *(const u16x8*)(kr + (int64_t)j * p.d + c8);
#pragma unroll
      for (int i = 0; i < 8; ++i) KT[(int64_t)(c8 + i) * b + j] = bf2f(x[i]);
    }
    return;
  }
  const int m0 = (blockIdx.x / ntn) * kT, n0 = (blockIdx.x % ntn) * kT;
  const Src B = {v.W0 + p.off[l], nin, nout};
  f32x16 acc[1] = {};
  if (l == 1)
    gemm1<128, false, true>(acc[0], Src{tok_rows(p.k, p, s, v.c0), p.d, n}, B, m0, n0, nin, stage_lds());
  else
    gemm1<128, true, true>(acc[0], Src{at<float>(v.reg, y.act[l - 1]), nin, n}, B, m0, n0, nin, stage_lds());
  const int col = acc_col(n0);
  float val[16];
  if (l < p.L) {
    float* act = at<float>(v.reg, y.act[l]);
    float* sp = at<float>(v.reg, y.sp[l]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(m0, r);
      const float z = acc[0][r];
      val[r] = silu(z);
      if (row < n) {
        act[(int64_t)row * nout + col] = val[r];
        sp[(int64_t)row * nout + col] = silu_prime(z);
      }
    }
    store_T(at<float>(v.reg, y.actT[l]), b, m0, n0, val);
  } else {
    const uint16_t* vr = tok_rows(p.v, p, s, v.c0);
    float* dl = at<float>(v.reg, y.dlt[l]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(m0, r);
      val[r] = acc[0][r] - bf2f(vr[(int64_t)min(row, n - 1) * p.d + col]);   // residual M(k) - v
      if (row < n) dl[(int64_t)row * nout + col] = val[r];
    }
    store_T(at<float>(v.reg, y.dltT[l]), b, m0, n0, val);
  }
}

// ---- backprop: delta^{l-1} = (delta^l W_0^l) * SiLU'(z^{l-1}) ----
__global__ void __launch_bounds__(kThreads) deep_back_kernel(DP p, int c, int l) {
  const int s = blockIdx.y;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nin / kT;
  const int m0 = (blockIdx.x / ntn) * kT, n0 = (blockIdx.x % ntn) * kT;
  const Src A = {at<float>(v.reg, y.dlt[l]), nout, n};
  const Src B = {v.WT0 + p.off[l], nout, nin};   // W^l transposed: [nin][nout]
  f32x16 acc[1] = {};
  gemm1<128, true, true>(acc[0], A, B, m0, n0, nout, stage_lds());
  const int col = acc_col(n0);
  const float* sp = at<float>(v.reg, y.sp[l - 1]);
  float* dl = l - 1 >= 2 ? at<float>(v.reg, y.dlt[l - 1]) : nullptr;
  float val[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    val[r] = acc[0][r] * sp[(int64_t)min(row, n - 1) * nin + col];
    if (dl && row < n) dl[(int64_t)row * nin + col] = val[r];
  }
  store_T(at<float>(v.reg, y.dltT[l - 1]), b, m0, n0, val);
}

// ---- fold of the chunk into the state, every layer in one launch: from
// slot c % 3 into slot (c + 1) % 3, or into (W_out, S_out) at the last chunk ----
__global__ void __launch_bounds__(kThreads) deep_fold_kernel(DP p, int c, int last) {
  __shared__ float wD[kMaxChunkDeep], wU[kMaxChunkDeep];
  const int s = blockIdx.y;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  int l = 1, t = blockIdx.x;
  while (l < p.L && t >= (p.w[l] / kT) * (p.w[l - 1] / kT)) {
    t -= (p.w[l] / kT) * (p.w[l - 1] / kT);
    ++l;
  }
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nin / kT;
  const int m0 = (t / ntn) * kT, n0 = (t % ntn) * kT;
  const float* cf = at<float>(v.reg, y.coef);
  for (int j = threadIdx.x; j < kMaxChunkDeep; j += kThreads) {
    wD[j] = j < n ? cf[4 * b + j] : 0.f;
    wU[j] = j < n ? cf[3 * b + j] : 0.f;
  }
  __syncthreads();
  const Src A = {at<float>(v.reg, y.dltT[l]), b, nout};
  const Src B[1] = {{at<float>(v.reg, y.actT[l - 1]), b, nin}};
  f32x16 g[2][1] = {};
  gemm<64, 2, 1, true, true, true>(g, A, B, m0, n0, n, wD, wU, stage_lds());
  const f32x16 acc[2] = {g[0][0], g[1][0]};
  const float An = cf[n - 1], En = cf[b + n - 1], Fn = cf[2 * b + n - 1];
  const float* Wsrc = v.W0 + p.off[l];
  const float* Ssrc = v.S0 + p.off[l];
  float* Wd = (last ? p.W + (int64_t)s * p.P : v.W1) + p.off[l];
  float* Sd = (last ? p.S + (int64_t)s * p.P : v.S1) + p.off[l];
  const int col = acc_col(n0);
  float wn[16], sn[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = (int64_t)acc_row(m0, r) * nin + col;
    const float w0 = Wsrc[i], s0 = Ssrc[i];
    wn[r] = An * w0 + Fn * s0 - acc[0][r];
    sn[r] = En * s0 - acc[1][r];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = (int64_t)acc_row(m0, r) * nin + col;
    Wd[i] = wn[r];
    Sd[i] = sn[r];
  }
  if (!last) store_T(v.WT1 + p.off[l], nout, m0, n0, wn);
}

// ---- reads: masked, decay-weighted scores D o (h a^{l-1 T}), lower triangle ----
__global__ void __launch_bounds__(kThreads) deep_scores_kernel(DP p, int c, int l) {
  const int s = blockIdx.y;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  const int nin = p.w[l - 1];
  const int ntn = (n + kT - 1) / kT;
  const int m0 = (blockIdx.x / ntn) * kT, n0 = (blockIdx.x % ntn) * kT;
  f32x16 acc[1] = {};
  if (n0 <= m0 + kT - 1) {   // tiles above the diagonal are zero
    if (l == 1)
      gemm1<128, false, false>(acc[0], Src{tok_rows(p.q, p, s, v.c0), p.d, n}, Src{tok_rows(p.k, p, s, v.c0), p.d, n},
                               m0, n0, nin, stage_lds());
    else
      gemm1<128, true, true>(acc[0], Src{at<float>(v.reg, y.hq[(l - 1) & 1]), p.maxw, n},
                             Src{at<float>(v.reg, y.act[l - 1]), nin, n}, m0, n0, nin, stage_lds());
  }
  const float* D = at<float>(v.reg, y.D);
  float* P = at<float>(v.reg, y.P);
  const int col = acc_col(n0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    P[(int64_t)row * b + col] = (col <= row && row < n && col < n) ? D[(int64_t)row * b + col] * acc[0][r] : 0.f;
  }
}

// ---- reads: zq^l = diag(A) h W_0^T + diag(F) h S_0^T - P delta^l, then SiLU
// (or y at the last layer); chunk-start reads take zq^l = h W_0^T ----
__global__ void __launch_bounds__(kThreads) deep_read_kernel(DP p, int c, int l) {
  const int s = blockIdx.y;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nout / kT;
  const int m0 = (blockIdx.x / ntn) * kT, n0 = (blockIdx.x % ntn) * kT;
  const bool raw = p.read_mode == TM_READ_AFTER_WRITE;
  // h W_0^T and h S_0^T share the staged h (one pipeline); the masked term
  // runs over the chunk's tokens
  f32x16 ws[1][2] = {}, at_ = {};
  const Src WS[2] = {{v.W0 + p.off[l], nin, nout}, {v.S0 + p.off[l], nin, nout}};
  const Src Wonly[1] = {WS[0]};
  f32x16 wo[1][1] = {};
  if (l == 1) {
    const Src H = {tok_rows(p.q, p, s, v.c0), p.d, n};
    if (raw)
      gemm<64, 1, 2, false, false, true>(ws, H, WS, m0, n0, nin, nullptr, nullptr, stage_lds());
    else
      gemm<128, 1, 1, false, false, true>(wo, H, Wonly, m0, n0, nin, nullptr, nullptr, stage_lds());
  } else {
    const Src H = {at<float>(v.reg, y.hq[(l - 1) & 1]), p.maxw, n};
    if (raw)
      gemm<64, 1, 2, false, true, true>(ws, H, WS, m0, n0, nin, nullptr, nullptr, stage_lds());
    else
      gemm<128, 1, 1, false, true, true>(wo, H, Wonly, m0, n0, nin, nullptr, nullptr, stage_lds());
  }
  if (raw)
    gemm1<64, true, true>(at_, Src{at<float>(v.reg, y.P), b, n}, Src{at<float>(v.reg, y.dltT[l]), b, nout}, m0, n0,
                          n, stage_lds());
  const f32x16 aw[1] = {raw ? ws[0][0] : wo[0][0]}, as[1] = {ws[0][1]};
  const float* cf = at<float>(v.reg, y.coef);
  const int col = acc_col(n0);
  const bool lastl = l == p.L;
  float* hn = at<float>(v.reg, y.hq[l & 1]);
  uint16_t* yo = p.y + ((int64_t)s * p.N + v.c0) * p.d;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    const int rc = min(row, n - 1);
    const float zq = raw ? cf[rc] * aw[0][r] + cf[2 * b + rc] * as[0][r] - at_[r] : aw[0][r];
    if (row < n) {
      if (lastl)
        yo[(int64_t)row * p.d + col] = f2bf(zq);
      else
        hn[(int64_t)row * p.maxw + col] = silu(zq);
    }
  }
}

// ---- the input state into slot 0: W, S and W^T per layer ----
__global__ void __launch_bounds__(kThreads) deep_convert_kernel(DP p) {
  const int s = blockIdx.y;
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= p.P) return;
  int l = 1;
  while (l < p.L && i4 >= p.off[l + 1]) ++l;
  const int nin = p.w[l - 1], nout = p.w[l];
  const int64_t e = i4 - p.off[l];
  const int r = (int)(e / nin), c4 = (int)(e % nin);
  unsigned char* base = p.ws + (int64_t)s * p.ws_stride + 2 * p.lay.region;
  float* W = (float*)base;
  float* S = (float*)(base + p.lay.copy);
  float* WT = (float*)(base + 2 * p.lay.copy);
  const float4 w = *(const float4*)(p.W_in + (int64_t)s * p.P + i4);
  const float4 x = *(const float4*)(p.S_in + (int64_t)s * p.P + i4);
  *(float4*)(W + i4) = w;
  *(float4*)(S + i4) = x;
  const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) WT[p.off[l] + (int64_t)(c4 + i) * nout + r] = wv[i];
}

DP make_dp(const Shape& s, int chunk) {
  DP p{};
  p.N = s.N;
  p.d = s.d;
  p.L = s.L;
  p.chunk = chunk;
  p.nch = (s.N + chunk - 1) / chunk;
  p.read_mode = s.read_mode;
  p.chunk_gates = s.chunk_gates;
  for (int l = 0; l <= s.L; ++l) p.w[l] = s.widths[l];
  for (int l = 1; l <= s.L; ++l) p.off[l] = s.off[l];
  p.P = s.P;
  p.maxw = s.maxw;
  p.lay = deep_layout(s, chunk);
  p.ws_stride = p.lay.total;
  return p;
}

}  // namespace

bool deep_supported(const Shape& s, int chunk) {
  if (s.io != TM_IO_BF16 || s.L < 2 || s.N <= 0) return false;
  if (chunk <= 0 || chunk > kMaxChunkDeep) return false;
  for (int l = 0; l <= s.L; ++l)
    if (s.widths[l] % kT != 0 || s.widths[l] > 4096) return false;
  return s.streams <= 65535;
}

int64_t deep_ws_bytes(const Shape& s, int chunk) { return deep_layout(s, chunk).total * (int64_t)s.streams; }

hipError_t launch_deep(const Shape& s, int chunk, const void* k, const void* v, const void* q, const float* alpha,
                       const float* eta, const float* theta, const float* W_in, const float* S_in, void* y,
                       float* W_out, float* S_out, void* ws, hipStream_t stream) {
  DP p = make_dp(s, chunk);
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.q = (const uint16_t*)q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.y = (uint16_t*)y;
  p.W_in = W_in;
  p.S_in = S_in;
  p.W = W_out;
  p.S = S_out;
  p.ws = (unsigned char*)ws;
  const int L = s.L;
  const int S = s.streams;
  hipError_t e;
  hipLaunchKernelGGL(deep_convert_kernel, dim3((unsigned)((s.P / 4 + kThreads - 1) / kThreads), S), dim3(kThreads),
                     0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  std::unique_lock<std::mutex> lock;
  SideStream* x = nullptr;
  if ((e = side_stream(dev, &x, lock)) != hipSuccess) return e;
  const bool raw = s.read_mode == TM_READ_AFTER_WRITE;
  auto chunks = [&]() -> hipError_t {
    hipError_t err;
    for (int c = 0; c < p.nch; ++c) {
      const int n = std::min(chunk, s.N - c * chunk);
      const int mt = (n + kT - 1) / kT;
      // the sweep of chunk c reuses region c % 2 and writes slot (c + 1) % 3,
      // both last read by the reads of chunk c - 2
      if (c >= 2 && (err = hipStreamWaitEvent(stream, x->cons[c & 1], 0)) != hipSuccess) return err;
      for (int l = 1; l <= L; ++l) {
        hipLaunchKernelGGL(deep_key_kernel, dim3(mt * (s.widths[l] / kT) + (l == 1), S), dim3(kThreads), 0, stream,
                           p, c, l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      for (int l = L; l >= 2; --l) {
        hipLaunchKernelGGL(deep_back_kernel, dim3(mt * (s.widths[l - 1] / kT), S), dim3(kThreads), 0, stream, p, c,
                           l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      if ((err = hipEventRecord(x->prod[c & 1], stream)) != hipSuccess) return err;
      if ((err = hipStreamWaitEvent(x->st, x->prod[c & 1], 0)) != hipSuccess) return err;
      for (int l = 1; l <= L; ++l) {
        if (raw) {
          hipLaunchKernelGGL(deep_scores_kernel, dim3(mt * mt, S), dim3(kThreads), 0, x->st, p, c, l);
          if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        hipLaunchKernelGGL(deep_read_kernel, dim3(mt * (s.widths[l] / kT), S), dim3(kThreads), 0, x->st, p, c, l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      if ((err = hipEventRecord(x->cons[c & 1], x->st)) != hipSuccess) return err;
      int tiles = 0;
      for (int l = 1; l <= L; ++l) tiles += (s.widths[l] / kT) * (s.widths[l - 1] / kT);
      hipLaunchKernelGGL(deep_fold_kernel, dim3(tiles, S), dim3(kThreads), 0, stream, p, c, c == p.nch - 1 ? 1 : 0);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
  };
  return join_side(x, stream, chunks());
}

}  // namespace titans
