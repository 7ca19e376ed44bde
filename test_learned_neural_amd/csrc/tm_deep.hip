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
// spread over the CUs:
//
//   sweep (caller's stream)  key(1) .. key(L), back(L) .. back(2), fold
//   reads (a second stream)  scores(1), read(1), .. scores(L), read(L)
//
// The reads of chunk c need the chunk-start state and the chunk's
// activations and deltas, not the fold, so they run beside the fold of
// chunk c and the sweep of chunk c + 1.  Every contraction runs on
// v_mfma_f32_32x32x16_bf16 with fp32 sums; its operands are staged through
// LDS in 64- or 128-deep k slices, the next slice's loads in flight while
// the current slice is multiplied.  The key, backprop and read products take
// 128 token rows per workgroup (eight waves), so each reads the chunk-start
// state once; the scores and the fold take 64 x 64 tiles (four waves).  Every
// tile of a stream runs on one XCD (place()).
//
// Precision: a product of two bf16-rounded operands carries about 2^-8 of
// error, and through four layers, the masked scores and the fold that sits
// at the edge of the 2e-2 bar (alpha = 1: 2.1e-2 per token).  So every
// operand but the exact bf16 keys and queries is split into hi = bf16(x) and
// lo = bf16(x - hi), and products are summed as hi*hi + hi*lo + lo*hi (three
// instructions, about 2^-16).  The producers write their results (a^l,
// delta^l, the query activations, the scores) as hi/lo pairs once; the
// fp32 state is split as it is staged.  Operands always have k contiguous in
// memory: the producers write a transposed copy where a later contraction
// runs over the tokens (a^l scaled by the fold weights D[n-1, .] and U,
// delta^l), and the backprop stages W^l transposed.
//
// The state stays fp32 and is read and written with non-temporal (streaming)
// loads and stores: it is touched once per chunk by each product, and kept
// out of L2 it leaves room there for the activations and deltas that a
// stream's tiles re-read.  The fold reads it from slot c % 3 of the workspace
// and writes the new state to slot (c + 1) % 3 (W_out / S_out at the last
// chunk); the chunk intermediates alternate between two regions.  So the
// reads of chunk c (slot c % 3, region c % 2) never meet the writes of the
// two chunks after it: the sweep of chunk c + 2 waits for the reads of chunk
// c before it starts.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace titans {
namespace {

constexpr int kT = 64;                 // output tile rows and columns
constexpr int kThreads = 256;          // four waves (64-row tiles)
constexpr int kMT = 128;               // token rows per tile of the key, backprop and read products
constexpr int kThreadsW = 4 * kMT;     // eight waves
constexpr int kMaxChunkDeep = 256;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// a 16-byte load that does not stay in the caches (the state, read once a chunk)
__device__ __forceinline__ float4 load_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

// A "pair" array holds each value x as hi = bf16(x) and lo = bf16(x - hi)
// (x - hi is exact in fp32): the hi plane, then the lo plane of the same
// shape, the bytes of an fp32 array.  A product of two pair operands is
// summed as hi*hi + hi*lo + lo*hi on the matrix cores with fp32 sums, about
// 2^-16 relative per product instead of bf16's 2^-8.  The producers write
// their results as pairs once; the contractions that re-read them stage
// the planes as they are.  The fp32 state is split as it is staged.
//
// Byte offsets in one stream's workspace.
struct DLayout {
  int b;   // token rows per region (the chunk rounded up to 64)
  int64_t act[kMaxLayers + 1];    // a^l [b][w_l] pair, l = 1..L-1
  int64_t actD[kMaxLayers + 1];   // D[n-1, j] a^l_j, transposed [w_l][b] pair, l = 0..L-1 (a^0 = K)
  int64_t actU[kMaxLayers + 1];   // U_j a^l_j, transposed [w_l][b] pair, l = 0..L-1
  int64_t sp[kMaxLayers + 1];     // SiLU'(z^l) [b][w_l] fp32, l = 1..L-1
  int64_t dlt[kMaxLayers + 1];    // delta^l [b][w_l] pair, l = 2..L
  int64_t dltT[kMaxLayers + 1];   // delta^l transposed [w_l][b] pair, l = 1..L
  int64_t hq[2];                  // query-side activations [b][maxw] pair, ping-pong
  int64_t P;                      // masked scores [b][b] pair
  int64_t D;                      // decay weights [b][b] fp32
  int64_t coef;                   // A, E, F, U, D[n-1, :]: [5][b] fp32
  int64_t region;                 // bytes per region
  int64_t copy;                   // bytes per fp32 state array (P floats, 256-byte aligned)
  int64_t slot;                   // bytes per slot: W and S
  int64_t total;                  // bytes per stream: two regions and three slots
};

int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

DLayout deep_layout(const Shape& s, int chunk) {
  DLayout y{};
  const int rows = chunk < s.N ? chunk : (s.N > 0 ? s.N : 1);
  y.b = (rows + kT - 1) / kT * kT;
  const int64_t b = y.b;
  int64_t cur = 0;
  auto take = [&](int64_t elems) {   // 4 bytes per element: fp32, or a pair's two planes
    const int64_t at = cur;
    cur += al256(elems * 4);
    return at;
  };
  for (int l = 1; l < s.L; ++l) y.act[l] = take(b * s.widths[l]);
  for (int l = 0; l < s.L; ++l) y.actD[l] = take(b * s.widths[l]);
  for (int l = 0; l < s.L; ++l) y.actU[l] = take(b * s.widths[l]);
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
  y.slot = 2 * y.copy;
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
  unsigned char* reg;          // this chunk's region
  const float *W0, *S0;        // chunk-start state (slot c % 3)
  float *W1, *S1;              // the fold's result (slot (c + 1) % 3)
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
  v.W1 = (float*)sw;
  v.S1 = (float*)(sw + p.lay.copy);
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

// An operand: element (row, k) at p[row * ld + k], k contiguous (kF32T:
// p[k * ld + row]); a pair's lo plane starts `lo` elements after p.  Rows at
// or past `rows` read row rows - 1 (an address in range) and count as zero,
// and so does every k >= K.  Loads stop at the first piece (4 fp32 or 8 bf16
// values) at or past K; a piece that straddles K reads up to K rounded up to
// 8, which every source's row holds (K a multiple of 64, or rows padded to a
// multiple of 64).
struct Src {
  const void* p;
  int64_t ld;
  int rows;
  int64_t lo;
};

enum Kind { kBF16, kF32, kPair, kF32T };   // exact bf16 input, fp32, pair, fp32 read transposed

template <int KS, int ROWS = kT>
__host__ __device__ constexpr int tile_elems() { return ROWS * (KS + 8); }

// Staging of one operand's 64 x KS slice into its hi (and lo) LDS tiles
// (row stride KS + 8 bf16).
template <Kind K, int KS, int ROWS, int NT>
struct Stage;

template <int KS, int ROWS, int NT>
struct Stage<kBF16, KS, ROWS, NT> {   // pieces of 8 values; hi only
  static constexpr int kQ = KS / 8, kPer = ROWS * kQ / NT, RS = KS + 8;
  uint4 r[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0, int K) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 8;
      r[u] = k0 + kq < K ? *(const uint4*)((const uint16_t*)a.p + (int64_t)min(r0 + row, a.rows - 1) * a.ld + k0 + kq)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* t, int rows_left, int k_left) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 8;
      const int kv = row < rows_left ? k_left - kq : 0;
      u16x8 x = __builtin_bit_cast(u16x8, r[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= kv) x[i] = 0;
      *(u16x8*)(t + row * RS + kq) = x;
    }
  }
};

template <int KS, int ROWS, int NT>
struct Stage<kPair, KS, ROWS, NT> {   // pieces of 8 values from each plane
  static constexpr int kQ = KS / 8, kPer = ROWS * kQ / NT, RS = KS + 8;
  uint4 h[kPer], l[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0, int K) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 8;
      const uint16_t* x = (const uint16_t*)a.p + (int64_t)min(r0 + row, a.rows - 1) * a.ld + k0 + kq;
      const bool in = k0 + kq < K;
      h[u] = in ? *(const uint4*)x : make_uint4(0u, 0u, 0u, 0u);
      l[u] = in ? *(const uint4*)(x + a.lo) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* t, int rows_left, int k_left) const {
    constexpr int TE = tile_elems<KS, ROWS>();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 8;
      const int kv = row < rows_left ? k_left - kq : 0;
      u16x8 xh = __builtin_bit_cast(u16x8, h[u]), xl = __builtin_bit_cast(u16x8, l[u]);
      if (kv < 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i >= kv) xh[i] = xl[i] = 0;
      }
      *(u16x8*)(t + row * RS + kq) = xh;
      *(u16x8*)(t + TE + row * RS + kq) = xl;
    }
  }
};

template <int KS, int ROWS, int NT>
struct Stage<kF32, KS, ROWS, NT> {   // pieces of 4 fp32 values, split as they are stored
  static constexpr int kQ = KS / 4, kPer = ROWS * kQ / NT, RS = KS + 8;
  float4 r[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0, int K) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 4;
      r[u] = k0 + kq < K ? load_stream((const float*)a.p + (int64_t)min(r0 + row, a.rows - 1) * a.ld + k0 + kq)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(uint16_t* t, int rows_left, int k_left) const {
    constexpr int TE = tile_elems<KS, ROWS>();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, row = e / kQ, kq = (e % kQ) * 4;
      const int kv = row < rows_left ? k_left - kq : 0;
      const float x[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
      u16x4 hv, lv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xi = i < kv ? x[i] : 0.f;
        hv[i] = f2bf(xi);
        lv[i] = f2bf(xi - bf2f(hv[i]));
      }
      *(u16x4*)(t + row * RS + kq) = hv;
      *(u16x4*)(t + TE + row * RS + kq) = lv;
    }
  }
};

template <int KS, int ROWS, int NT>
struct Stage<kF32T, KS, ROWS, NT> {   // fp32 read transposed: pieces of 4 rows at one k, split as they are stored
  static constexpr int kQ = ROWS / 4, kPer = KS * kQ / NT, RS = KS + 8;
  float4 r[kPer];
  __device__ __forceinline__ void fetch(const Src& a, int r0, int k0, int K) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, k = e / kQ, rq = (e % kQ) * 4;
      r[u] = k0 + k < K ? load_stream((const float*)a.p + (int64_t)(k0 + k) * a.ld + r0 + rq)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(uint16_t* t, int rows_left, int k_left) const {
    constexpr int TE = tile_elems<KS, ROWS>();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * NT, k = e / kQ, rq = (e % kQ) * 4;
      const float x[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xi = (rq + i < rows_left && k < k_left) ? x[i] : 0.f;
        const unsigned short hv = f2bf(xi);
        t[(rq + i) * RS + k] = hv;
        t[TE + (rq + i) * RS + k] = f2bf(xi - bf2f(hv));
      }
    }
  }
};

__host__ __device__ constexpr bool has_lo(Kind k) { return k != kBF16; }

// acc[t] += A(m0 + i, k) B_t(n0 + j, k) summed over k < K, for the wave's
// 32 x 32 block (i in [0, MT), j in [0, 64)), as one pipeline: the next
// KS-deep slice's loads are in flight while the current slice is multiplied.
// MT / 16 waves (MT x 4 threads) cover the MT x 64 tile, wave w the block at
// row 32 (w / 2), column 32 (w % 2).  The NB operands B_t share the staged
// A.  LDS tiles: A hi, A lo (MT rows), then B_t hi, lo (64 rows).
// v_mfma_f32_32x32x16_bf16: lane l supplies row (A) or column (B) l % 32 with
// k values 8 (l / 32) .. + 7 of each 16-deep step; accumulator register r of
// lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
template <int KS, int NB, Kind AK, Kind BK, int MT = kT>
__device__ void gemm(f32x16 (&acc)[NB], const Src A, const Src (&B)[NB], int m0, int n0, int K, uint16_t* lds) {
  constexpr int NT = 4 * MT, RS = KS + 8;
  constexpr int TA = tile_elems<KS, MT>(), TB = tile_elems<KS>();
  constexpr bool alo = has_lo(AK), blo = has_lo(BK);
  uint16_t* const As = lds;
  uint16_t* const Bs = lds + 2 * TA;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = (wv >> 1) * 32, wn = (wv & 1) * 32;
  Stage<AK, KS, MT, NT> sa;
  Stage<BK, KS, kT, NT> sb[NB];
  if (K <= 0) return;
  sa.fetch(A, m0, 0, K);
#pragma unroll
  for (int t = 0; t < NB; ++t) sb[t].fetch(B[t], n0, 0, K);
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int t = 0; t < NB; ++t) sb[t].store(Bs + 2 * t * TB, B[t].rows - n0, K - k0);
    sa.store(As, A.rows - m0, K - k0);
    __syncthreads();
    if (k0 + KS < K) {
      sa.fetch(A, m0, k0 + KS, K);
#pragma unroll
      for (int t = 0; t < NB; ++t) sb[t].fetch(B[t], n0, k0 + KS, K);
    }
#pragma unroll
    for (int kk = 0; kk < KS; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      const uint16_t* ar = As + (wm + (lane & 31)) * RS + ko;
      const bf16x8 ah = *(const bf16x8*)ar;
      bf16x8 al;
      if constexpr (alo) al = *(const bf16x8*)(ar + TA);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const uint16_t* br = Bs + 2 * t * TB + (wn + (lane & 31)) * RS + ko;
        const bf16x8 bh = *(const bf16x8*)br;
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[t], 0, 0, 0);
        if constexpr (blo) {
          const bf16x8 bl = *(const bf16x8*)(br + TB);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[t], 0, 0, 0);
        }
        if constexpr (alo) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
}

template <int KS, Kind AK, Kind BK, int MT = kT>
__device__ __forceinline__ void gemm1(f32x16& acc, const Src A, const Src B, int m0, int n0, int K, uint16_t* lds) {
  f32x16 a[1] = {acc};
  const Src b[1] = {B};
  gemm<KS, 1, AK, BK, MT>(a, A, b, m0, n0, K, lds);
  acc = a[0];
}

// (stream, tile) of this workgroup in a one-dimensional grid of T tiles for
// each of the launch's streams.  Consecutive workgroups go to the eight XCDs
// in turn; when the stream count is a multiple of 8, every tile of a stream
// lands on one XCD (streams s, s + 8, ... on XCD s % 8, tile after tile), so
// the operands its tiles share come from that XCD's L2 after the first read.
struct Place {
  int s, tile;
};
__device__ __forceinline__ Place place(int T) {
  const int id = blockIdx.x, S = gridDim.x / T;
  if ((S & 7) == 0) {
    const int j = id >> 3;
    return Place{(id & 7) + 8 * (j / T), j % T};
  }
  return Place{id / T, id % T};
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

// x as a pair at element i of the array whose lo plane starts lo after it
__device__ __forceinline__ void put_pair(uint16_t* a, int64_t lo, int64_t i, float x) {
  const unsigned short h = f2bf(x);
  a[i] = h;
  a[lo + i] = f2bf(x - bf2f(h));
}

// The tile transposed into a pair array: T[col][row .. row + 3] from
// registers 4g .. 4g + 3 (four consecutive rows), each scaled by w[row - m0]
// when w is given (LDS), one 8-byte store per plane and group.  T's rows
// hold ldT tokens (a multiple of 64); groups at or past them are skipped.
__device__ __forceinline__ void store_T(uint16_t* T, int64_t lo, int64_t ldT, int m0, int n0, const float (&v)[16],
                                        const float* w = nullptr) {
  const int col = acc_col(n0);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int row = acc_row(m0, 4 * g);
    if (row >= ldT) continue;
    u16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = w ? v[4 * g + i] * w[row - m0 + i] : v[4 * g + i];
      h[i] = f2bf(x);
      l[i] = f2bf(x - bf2f(h[i]));
    }
    *(u16x4*)(T + (int64_t)col * ldT + row) = h;
    *(u16x4*)(T + lo + (int64_t)col * ldT + row) = l;
  }
}

__device__ __forceinline__ const uint16_t* tok_rows(const uint16_t* base, const DP& p, int s, int c0) {
  return base + ((int64_t)s * p.N + c0) * p.d;
}

// The staging area every contraction of a kernel shares, E bf16 elements
// (one allocation per size): the key, backprop and read kernels hold hi and
// lo of a 128-row A and one 64-row B 128 deep (or of two B 64 deep), the
// scores kernel of a 64-row A and one B 128 deep, the fold of a 64-row A and
// two B 64 deep.
constexpr int kLdsW = 2 * tile_elems<128, kMT>() + 2 * tile_elems<128>();
constexpr int kLdsScores = 4 * tile_elems<128>();
constexpr int kLdsFold = 6 * tile_elems<64>();
static_assert(kLdsW >= 2 * tile_elems<64, kMT>() + 4 * tile_elems<64>(), "read kernel staging");
template <int E>
__device__ __forceinline__ uint16_t* stage_lds() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[E];
  return buf;
}

// pair arrays of the region: pointer and lo-plane offset (elements)
struct PairArr {
  uint16_t* p;
  int64_t lo;
};
__device__ __forceinline__ PairArr pair(unsigned char* reg, int64_t off, int64_t elems) {
  return PairArr{at<uint16_t>(reg, off), elems};
}

// The fold weights D[n-1, i] and U_i of tokens m0 .. m0 + kMT - 1 of chunk
// c (zero past the chunk's n tokens) into w[0, kMT) and w[kMT, 2 kMT): the
// gates of the chunk's later tokens go through LDS, then one thread per
// token runs its column's recurrence over them.
__device__ void fold_weights(const DP& p, int s, int c, int n, int m0, float* w) {
  __shared__ float ga[kMaxChunkDeep], ge[kMaxChunkDeep], gt[kMaxChunkDeep];
  const int t = threadIdx.x;
  const int64_t g0 = p.chunk_gates ? (int64_t)s * p.nch + c : (int64_t)s * p.N + (int64_t)c * p.chunk;
  const int gs = p.chunk_gates ? 0 : 1;
  for (int j = m0 + t; j < n; j += blockDim.x) {
    ga[j] = p.alpha[g0 + j * gs];
    ge[j] = p.eta[g0 + j * gs];
    gt[j] = p.theta[g0 + j * gs];
  }
  __syncthreads();
  if (t < kMT) {
    const int i = m0 + t;
    float di = 0.f, u = 0.f;
    if (i < n) {
      const float ti = gt[i];
      float pr = 1.f;
      di = ti;
      for (int j = i + 1; j < n; ++j) {
        pr *= ge[j];
        di = (1.f - ga[j]) * di + ti * pr;
      }
      u = ti * pr;
    }
    w[t] = di;
    w[kMT + t] = u;
  }
  __syncthreads();
}

// ---- key side: z^l = a^{l-1} W_0^l^T (and, in layer 1's extra workgroup
// per stream, the chunk's coefficients and the scaled transposed keys) ----
__global__ void __launch_bounds__(kThreadsW) deep_key_kernel(DP p, int c, int l) {
  const int n = min(p.chunk, p.N - c * p.chunk);
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nout / kT, ntiles = ((n + kMT - 1) / kMT) * ntn;
  const Place pl = place(ntiles + (l == 1));
  const int s = pl.s;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b;
  if (pl.tile >= ntiles) {
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
      float di = 0.f, pr = 1.f, ui = 0.f;
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
        ui = ti * pr;
      } else {
        for (int j = 0; j < b; ++j) D[(int64_t)j * b + i] = 0.f;
        di = 0.f;
      }
      cf[3 * b + i] = ui;   // U
      cf[4 * b + i] = di;   // D[n-1, i]
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
    return;
  }
  const int m0 = (pl.tile / ntn) * kMT, n0 = (pl.tile % ntn) * kT;
  const Src B = {v.W0 + p.off[l], nin, nout, 0};
  f32x16 acc = {};
  if (l == 1)
    gemm1<128, kBF16, kF32, kMT>(acc, Src{tok_rows(p.k, p, s, v.c0), p.d, n, 0}, B, m0, n0, nin, stage_lds<kLdsW>());
  else
    gemm1<128, kPair, kF32, kMT>(acc, Src{at<uint16_t>(v.reg, y.act[l - 1]), nin, n, (int64_t)b * nin}, B, m0, n0,
                                 nin, stage_lds<kLdsW>());
  const int col = acc_col(n0);
  float val[16];
  if (l < p.L) {
    __shared__ float w[2 * kMT];
    if (l == 1) {
      fold_weights(p, s, c, n, m0, w);
    } else {
      const float* cf = at<float>(v.reg, y.coef);
      if (threadIdx.x < kMT) {
        const int i = min(m0 + (int)threadIdx.x, b - 1);
        w[threadIdx.x] = cf[4 * b + i];
        w[kMT + threadIdx.x] = cf[3 * b + i];
      }
      __syncthreads();
    }
    const PairArr act = pair(v.reg, y.act[l], (int64_t)b * nout);
    float* sp = at<float>(v.reg, y.sp[l]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(m0, r);
      const float z = acc[r];
      val[r] = silu(z);
      if (row < n) {
        put_pair(act.p, act.lo, (int64_t)row * nout + col, val[r]);
        sp[(int64_t)row * nout + col] = silu_prime(z);
      }
    }
    const PairArr aD = pair(v.reg, y.actD[l], (int64_t)nout * b), aU = pair(v.reg, y.actU[l], (int64_t)nout * b);
    store_T(aD.p, aD.lo, b, m0, n0, val, w);
    store_T(aU.p, aU.lo, b, m0, n0, val, w + kMT);
    if (l == 1 && n0 == 0) {
      // the keys of these kMT tokens, scaled by the fold weights, into K^T
      // [d][b] pairs for the fold's contraction over tokens (consecutive
      // tokens along each row of K^T, so the stores are whole rows)
      const uint16_t* kr = tok_rows(p.k, p, s, v.c0);
      const PairArr KD = pair(v.reg, y.actD[0], (int64_t)p.d * b), KU = pair(v.reg, y.actU[0], (int64_t)p.d * b);
      const int rows = min(kMT, b - m0);
      for (int e = threadIdx.x; e < rows * p.d; e += kThreadsW) {
        const int j = e % rows, cc = e / rows;
        const float x = bf2f(kr[(int64_t)min(m0 + j, n - 1) * p.d + cc]);
        put_pair(KD.p, KD.lo, (int64_t)cc * b + m0 + j, w[j] * x);
        put_pair(KU.p, KU.lo, (int64_t)cc * b + m0 + j, w[kMT + j] * x);
      }
    }
  } else {
    const uint16_t* vr = tok_rows(p.v, p, s, v.c0);
    const PairArr dl = pair(v.reg, y.dlt[l], (int64_t)b * nout), dT = pair(v.reg, y.dltT[l], (int64_t)nout * b);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(m0, r);
      val[r] = acc[r] - bf2f(vr[(int64_t)min(row, n - 1) * p.d + col]);   // residual M(k) - v
      if (row < n) put_pair(dl.p, dl.lo, (int64_t)row * nout + col, val[r]);
    }
    store_T(dT.p, dT.lo, b, m0, n0, val);
  }
}

// ---- backprop: delta^{l-1} = (delta^l W_0^l) * SiLU'(z^{l-1}) ----
__global__ void __launch_bounds__(kThreadsW) deep_back_kernel(DP p, int c, int l) {
  const int n = min(p.chunk, p.N - c * p.chunk);
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nin / kT;
  const Place pl = place(((n + kMT - 1) / kMT) * ntn);
  const int s = pl.s;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b;
  const int m0 = (pl.tile / ntn) * kMT, n0 = (pl.tile % ntn) * kT;
  // B(c, r) = W^l[r][c], staged transposed from W^l [nout][nin]
  f32x16 acc = {};
  gemm1<128, kPair, kF32T, kMT>(acc, Src{at<uint16_t>(v.reg, y.dlt[l]), nout, n, (int64_t)b * nout},
                                Src{v.W0 + p.off[l], nin, nin, 0}, m0, n0, nout, stage_lds<kLdsW>());
  const int col = acc_col(n0);
  const float* sp = at<float>(v.reg, y.sp[l - 1]);
  const PairArr dl = pair(v.reg, y.dlt[l - 1], (int64_t)b * nin), dT = pair(v.reg, y.dltT[l - 1], (int64_t)nin * b);
  float val[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    val[r] = acc[r] * sp[(int64_t)min(row, n - 1) * nin + col];
    if (l - 1 >= 2 && row < n) put_pair(dl.p, dl.lo, (int64_t)row * nin + col, val[r]);
  }
  store_T(dT.p, dT.lo, b, m0, n0, val);
}

// ---- fold of the chunk into the state, every layer in one launch: from
// slot c % 3 into slot (c + 1) % 3, or into (W_out, S_out) at the last chunk ----
__global__ void __launch_bounds__(kThreads) deep_fold_kernel(DP p, int c, int last) {
  int T = 0;
  for (int l = 1; l <= p.L; ++l) T += (p.w[l] / kT) * (p.w[l - 1] / kT);
  const Place pl = place(T);
  const int s = pl.s;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b, n = v.n;
  int l = 1, t = pl.tile;
  while (l < p.L && t >= (p.w[l] / kT) * (p.w[l - 1] / kT)) {
    t -= (p.w[l] / kT) * (p.w[l - 1] / kT);
    ++l;
  }
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nin / kT;
  const int m0 = (t / ntn) * kT, n0 = (t % ntn) * kT;
  const int col = acc_col(n0);
  const float* Wsrc = v.W0 + p.off[l];
  const float* Ssrc = v.S0 + p.off[l];
  // the state tile's loads go out before the contraction
  float w0[16], s0[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = (int64_t)acc_row(m0, r) * nin + col;
    w0[r] = __builtin_nontemporal_load(Wsrc + i);
    s0[r] = __builtin_nontemporal_load(Ssrc + i);
  }
  // G(D[n-1, :]) and G(U): the deltas against the keys' activations scaled per token
  const Src B[2] = {{at<uint16_t>(v.reg, y.actD[l - 1]), b, nin, (int64_t)nin * b},
                    {at<uint16_t>(v.reg, y.actU[l - 1]), b, nin, (int64_t)nin * b}};
  f32x16 g[2] = {};
  gemm<64, 2, kPair, kPair>(g, Src{at<uint16_t>(v.reg, y.dltT[l]), b, nout, (int64_t)nout * b}, B, m0, n0, n,
                            stage_lds<kLdsFold>());
  const float* cf = at<float>(v.reg, y.coef);
  const float An = cf[n - 1], En = cf[b + n - 1], Fn = cf[2 * b + n - 1];
  float* Wd = (last ? p.W + (int64_t)s * p.P : v.W1) + p.off[l];
  float* Sd = (last ? p.S + (int64_t)s * p.P : v.S1) + p.off[l];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = (int64_t)acc_row(m0, r) * nin + col;
    __builtin_nontemporal_store(An * w0[r] + Fn * s0[r] - g[0][r], Wd + i);
    __builtin_nontemporal_store(En * s0[r] - g[1][r], Sd + i);
  }
}

// ---- reads: masked, decay-weighted scores D o (h a^{l-1 T}), lower triangle ----
__global__ void __launch_bounds__(kThreads) deep_scores_kernel(DP p, int c, int l) {
  const int n = min(p.chunk, p.N - c * p.chunk);
  const int nin = p.w[l - 1];
  const int ntn = (n + kT - 1) / kT;
  const Place pl = place(ntn * ntn);
  const int s = pl.s;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b;
  const int m0 = (pl.tile / ntn) * kT, n0 = (pl.tile % ntn) * kT;
  f32x16 acc = {};
  if (n0 <= m0 + kT - 1) {   // tiles above the diagonal are zero
    if (l == 1)
      gemm1<128, kBF16, kBF16>(acc, Src{tok_rows(p.q, p, s, v.c0), p.d, n, 0}, Src{tok_rows(p.k, p, s, v.c0), p.d, n, 0},
                               m0, n0, nin, stage_lds<kLdsScores>());
    else
      gemm1<128, kPair, kPair>(acc, Src{at<uint16_t>(v.reg, y.hq[(l - 1) & 1]), p.maxw, n, (int64_t)b * p.maxw},
                               Src{at<uint16_t>(v.reg, y.act[l - 1]), nin, n, (int64_t)b * nin}, m0, n0, nin,
                               stage_lds<kLdsScores>());
  }
  const float* D = at<float>(v.reg, y.D);
  const PairArr P = pair(v.reg, y.P, (int64_t)b * b);
  const int col = acc_col(n0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    put_pair(P.p, P.lo, (int64_t)row * b + col,
             (col <= row && row < n && col < n) ? D[(int64_t)row * b + col] * acc[r] : 0.f);
  }
}

// ---- reads: zq^l = diag(A) h W_0^T + diag(F) h S_0^T - P delta^l, then SiLU
// (or y at the last layer); chunk-start reads take zq^l = h W_0^T ----
__global__ void __launch_bounds__(kThreadsW) deep_read_kernel(DP p, int c, int l) {
  const int n = min(p.chunk, p.N - c * p.chunk);
  const int nin = p.w[l - 1], nout = p.w[l];
  const int ntn = nout / kT;
  const Place pl = place(((n + kMT - 1) / kMT) * ntn);
  const int s = pl.s;
  const View v = view(p, s, c);
  const DLayout& y = p.lay;
  const int b = y.b;
  const int m0 = (pl.tile / ntn) * kMT, n0 = (pl.tile % ntn) * kT;
  const bool raw = p.read_mode == TM_READ_AFTER_WRITE;
  // h W_0^T and h S_0^T share the staged h (one pipeline); the masked term
  // runs over the chunk's tokens
  f32x16 ws[2] = {}, wo[1] = {}, tk = {};
  const Src WS[2] = {{v.W0 + p.off[l], nin, nout, 0}, {v.S0 + p.off[l], nin, nout, 0}};
  const Src Wonly[1] = {WS[0]};
  if (l == 1) {
    const Src H = {tok_rows(p.q, p, s, v.c0), p.d, n, 0};
    if (raw)
      gemm<64, 2, kBF16, kF32, kMT>(ws, H, WS, m0, n0, nin, stage_lds<kLdsW>());
    else
      gemm<128, 1, kBF16, kF32, kMT>(wo, H, Wonly, m0, n0, nin, stage_lds<kLdsW>());
  } else {
    const Src H = {at<uint16_t>(v.reg, y.hq[(l - 1) & 1]), p.maxw, n, (int64_t)b * p.maxw};
    if (raw)
      gemm<64, 2, kPair, kF32, kMT>(ws, H, WS, m0, n0, nin, stage_lds<kLdsW>());
    else
      gemm<128, 1, kPair, kF32, kMT>(wo, H, Wonly, m0, n0, nin, stage_lds<kLdsW>());
  }
  if (raw)
    gemm1<64, kPair, kPair, kMT>(tk, Src{at<uint16_t>(v.reg, y.P), b, n, (int64_t)b * b},
                                 Src{at<uint16_t>(v.reg, y.dltT[l]), b, nout, (int64_t)nout * b}, m0, n0, n,
                                 stage_lds<kLdsW>());
  const float* cf = at<float>(v.reg, y.coef);
  const int col = acc_col(n0);
  const bool lastl = l == p.L;
  const PairArr hn = pair(v.reg, y.hq[l & 1], (int64_t)b * p.maxw);
  uint16_t* yo = p.y + ((int64_t)s * p.N + v.c0) * p.d;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(m0, r);
    const int rc = min(row, n - 1);
    const float zq = raw ? cf[rc] * ws[0][r] + cf[2 * b + rc] * ws[1][r] - tk[r] : wo[0][r];
    if (row < n) {
      if (lastl)
        yo[(int64_t)row * p.d + col] = f2bf(zq);
      else
        put_pair(hn.p, hn.lo, (int64_t)row * p.maxw + col, silu(zq));
    }
  }
}

// ---- the input state into slot 0 ----
__global__ void __launch_bounds__(kThreads) deep_convert_kernel(DP p) {
  const int s = blockIdx.y;
  const int64_t i4 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i4 >= p.P) return;
  unsigned char* base = p.ws + (int64_t)s * p.ws_stride + 2 * p.lay.region;
  *(float4*)((float*)base + i4) = *(const float4*)(p.W_in + (int64_t)s * p.P + i4);
  *(float4*)((float*)(base + p.lay.copy) + i4) = *(const float4*)(p.S_in + (int64_t)s * p.P + i4);
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
  // one-dimensional grids of tiles x streams (the input copy: streams in y)
  const int64_t mt = ((chunk < s.N ? chunk : s.N) + kT - 1) / kT;
  int64_t tiles = mt * mt;
  int64_t fold = 0;
  for (int l = 1; l <= s.L; ++l) {
    tiles = std::max<int64_t>(tiles, mt * (s.widths[l] / kT) + 1);
    fold += (int64_t)(s.widths[l] / kT) * (s.widths[l - 1] / kT);
  }
  tiles = std::max(tiles, fold);
  return s.streams <= 65535 && (int64_t)s.streams * tiles < ((int64_t)1 << 31);
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
      const int mt = (n + kT - 1) / kT, mw = (n + kMT - 1) / kMT;
      // the sweep of chunk c reuses region c % 2 and writes slot (c + 1) % 3,
      // both last read by the reads of chunk c - 2
      if (c >= 2 && (err = hipStreamWaitEvent(stream, x->cons[c & 1], 0)) != hipSuccess) return err;
      for (int l = 1; l <= L; ++l) {
        hipLaunchKernelGGL(deep_key_kernel, dim3((mw * (s.widths[l] / kT) + (l == 1)) * S), dim3(kThreadsW), 0, stream,
                           p, c, l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      for (int l = L; l >= 2; --l) {
        hipLaunchKernelGGL(deep_back_kernel, dim3(mw * (s.widths[l - 1] / kT) * S), dim3(kThreadsW), 0, stream, p, c,
                           l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      if ((err = hipEventRecord(x->prod[c & 1], stream)) != hipSuccess) return err;
      if ((err = hipStreamWaitEvent(x->st, x->prod[c & 1], 0)) != hipSuccess) return err;
      for (int l = 1; l <= L; ++l) {
        if (raw) {
          hipLaunchKernelGGL(deep_scores_kernel, dim3(mt * mt * S), dim3(kThreads), 0, x->st, p, c, l);
          if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        hipLaunchKernelGGL(deep_read_kernel, dim3(mw * (s.widths[l] / kT) * S), dim3(kThreadsW), 0, x->st, p, c, l);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      if ((err = hipEventRecord(x->cons[c & 1], x->st)) != hipSuccess) return err;
      int tiles = 0;
      for (int l = 1; l <= L; ++l) tiles += (s.widths[l] / kT) * (s.widths[l - 1] / kT);
      hipLaunchKernelGGL(deep_fold_kernel, dim3(tiles * S), dim3(kThreads), 0, stream, p, c, c == p.nch - 1 ? 1 : 0);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
  };
  return join_side(x, stream, chunks());
}

}  // namespace titans
