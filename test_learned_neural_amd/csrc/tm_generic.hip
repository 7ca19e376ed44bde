// Shape-generic fp32 kernel of the Titans memory hot path.
//
// One workgroup per (batch, head) stream walks the chunks in order.  Per
// chunk it evaluates the chunked form of "Titans: Learning to Memorize at
// Test Time" (mer.dev notes, section 3.2: every gradient of the chunk is
// taken at the chunk-start weights W_0) in closed form:
//
//   a1  coefficients from the gates (section 3.1 rules unrolled over the chunk)
//         A_j = prod_{m<=j} (1 - alpha_m)     E_j = prod_{m<=j} eta_m
//         F_j = (1 - alpha_j) F_{j-1} + E_j   U_i = theta_i prod_{m>i} eta_m
//         D[j,i] = (1 - alpha_j) D[j-1,i] + theta_i prod_{i<m<=j} eta_m,  D[i,i] = theta_i
//       so that W_j = A_j W_0 + F_j S_0 - sum_{i<=j} D[j,i] g_i and
//       S_n = E_n S_0 - sum_i U_i g_i, with g_i = delta_i a_i^T per layer.
//   a2  key-side forward at W_0:  z^l = a^{l-1} W_0^l^T, a^l = SiLU(z^l)
//   a3  residual and backprop:    delta^L = a^L - V,
//                                 delta^{l-1} = (delta^l W_0^l) * SiLU'(z^{l-1})
//   a5  retrieval after each token's write, layer by layer (h^0 = Q):
//         zq^l = diag(A) h W_0^T + diag(F) h S_0^T - (D o (h a^{l-1 T})) delta^l
//   a4  state update: W <- A_n W_0 + F_n S_0 - G(D[n-1,:]),  S <- E_n S_0 - G(U)
//         with G(w) = sum_j w_j delta_j a_j^T
//
// The state lives in W_out/S_out (global memory) and the chunk's
// intermediates in a per-stream workspace; every contraction is an fp32
// matrix-instruction tile loop staged through LDS.  This path serves any
// shape (the linear memory up to d = 64 goes to the one-workgroup kernel of
// tm_linear.hip instead), and is the fallback where no specialised kernel
// exists.
//
// A state too large for LDS leaves most CUs idle with one workgroup per
// stream; there the forward call runs each chunk in two phases: the sweep
// (a1-a4, on the caller's stream) and the reads (a5, on a second stream),
// which depend on the chunk-start state but not on the fold, so the reads of
// chunk c run beside the sweep of chunk c + 1.  The chunk-start states
// rotate through three buffers (the last one is W_out/S_out) and the chunk's
// intermediates through two workspace regions.  With few streams (at most a
// quarter as many as CUs) every step of a phase is a launch of its own, its
// contraction's output tiles spread over several workgroups per stream.
#include "tm_internal.h"
#include "tm_block_gemm.h"

#include <hip/hip_bf16.h>

#include <algorithm>
#include <mutex>

namespace titans {
namespace {

constexpr int kThreads = kGemmThreads;

// Per-stream workspace of the chunked sweep, as float offsets (computed on
// the host, read from the kernel arguments with scalar loads):
//   act[l]   a^l of the chunk's keys, [b x n_l] (a^0 = K)
//   sp[l]    SiLU'(z^l), l = 1..L-1;  delta[l]  delta^l, l = 1..L
//   vin      V [b x d];  hq[0..1]  query-side activations, ping-pong [b x maxw]
//   sc, D    masked scores and decay weights [b x b];  A, E, F, U  [b]
struct WsLayout {
  int64_t act[kMaxLayers + 1], sp[kMaxLayers + 1], delta[kMaxLayers + 1];
  int64_t vin, hq[2], sc, D, A, E, F, U;
  int64_t total;
};

WsLayout ws_layout(const Shape& s, int b) {
  WsLayout w{};
  int64_t cur = 0;
  for (int l = 0; l <= s.L; ++l) { w.act[l] = cur; cur += (int64_t)b * s.widths[l]; }
  for (int l = 1; l < s.L; ++l) { w.sp[l] = cur; cur += (int64_t)b * s.widths[l]; }
  for (int l = 1; l <= s.L; ++l) { w.delta[l] = cur; cur += (int64_t)b * s.widths[l]; }
  w.vin = cur; cur += (int64_t)b * s.d;
  w.hq[0] = cur; cur += (int64_t)b * s.maxw;
  w.hq[1] = cur; cur += (int64_t)b * s.maxw;
  w.sc = cur; cur += (int64_t)b * b;
  w.D = cur; cur += (int64_t)b * b;
  w.A = cur; cur += b;
  w.E = cur; cur += b;
  w.F = cur; cur += b;
  w.U = cur; cur += b;
  w.total = (cur + 63) / 64 * 64;                                     // keep 256-byte alignment
  return w;
}

struct GParams {
  int N, d, L, io, read_mode, chunk;
  int chunk_gates;   // gates hold one value per chunk
  int widths[kMaxLayers + 1];
  int64_t off[kMaxLayers + 1];
  int64_t P;
  int maxw;
  int b;  // rows reserved per chunk in the workspace
  const void* k;
  const void* v;
  const void* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  const float* W_in;
  const float* S_in;
  void* y;            // NULL: no retrieval (the state sweep only)
  float* W;
  float* S;
  int64_t state_stride;   // floats between streams in W, S (P unless they live in another layout)
  int64_t in_stride;      // floats between streams in W_in, S_in
  float* ckpt;        // optional: (W, S) at every chunk start, [chunk][W | S] per stream
  int64_t ckpt_stride;    // floats between streams in ckpt
  float* ws;
  int64_t ws_stride;  // floats per stream
  WsLayout lay;
  int lds_state;      // 1: the state and the workspace live in LDS for the whole sweep
  int64_t P4;         // P rounded up to a multiple of 4 (LDS layout: W, S, workspace)
  int64_t region;     // floats between the two workspace regions of the per-chunk launches
};

enum { kSweep = 1, kReads = 2, kBoth = 3 };
// One stage per launch (stage != kAllStages): the chunk's inputs and
// coefficients, or one contraction of one layer, its output tiles shared out
// over the launch's y dimension.
enum { kAllStages = 0, kLoad, kKey, kBack, kScores, kRead, kFoldW, kFoldS };

// Small problems keep the state (W, S) and the chunk workspace in LDS for the
// whole sweep, copied in at the start and out at the end: every contraction
// then reads and writes LDS instead of global memory.  Budget for that
// dynamic LDS, beside the contractions' own staging area.
constexpr int64_t kLdsStateBytes = 120 * 1024;

__device__ __forceinline__ float logistic(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float silu(float z) { return z * logistic(z); }
__device__ __forceinline__ float silu_prime(float z) {
  float s = logistic(z);
  return s * (1.0f + z * (1.0f - s));
}

__device__ __forceinline__ float load_io(const void* p, int64_t i, int io) {
  if (io == TM_IO_BF16) return __bfloat162float(((const __hip_bfloat16*)p)[i]);
  return ((const float*)p)[i];
}

__device__ __forceinline__ void store_io(void* p, int64_t i, float x, int io) {
  if (io == TM_IO_BF16)
    ((__hip_bfloat16*)p)[i] = __float2bfloat16(x);  // round to nearest even
  else
    ((float*)p)[i] = x;
}


// cs < 0: every chunk in order, the state folded in place in (W, S) after a
// copy from (W_in, S_in).  cs >= 0: chunk cs only, its start state read from
// (W_in, S_in) and the folded state written to (W, S); `phase` selects the
// sweep (a1-a4) and/or the reads (a5), `stage` and `layer` one step of them.
__global__ void __launch_bounds__(kThreads) generic_kernel(GParams p, int cs, int phase, int stage, int layer) {
  extern __shared__ __attribute__((aligned(16))) float dyn_lds[];
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = p.d, L = p.L;
  const bool one = cs >= 0;
  const bool sweep = phase & kSweep, rd = (phase & kReads) && p.y;
  float* const Wg = p.W + (int64_t)s * p.state_stride;
  float* const Sg = p.S + (int64_t)s * p.state_stride;
  const float* Win = p.W_in + (int64_t)s * p.in_stride;
  const float* Sin = p.S_in + (int64_t)s * p.in_stride;
  const bool in_lds = p.lds_state && p.N > 0;   // (never with one chunk per launch)
  float* const W = in_lds ? dyn_lds : Wg;
  float* const S = in_lds ? dyn_lds + p.P4 : Sg;
  const float* const Wr = one ? Win : W;   // the chunk-start state this launch reads
  const float* const Sr = one ? Sin : S;
  if (!one) {
    if (W != Win) each((int)p.P, [&](int i) { return Win[i]; }, [&](int i, float x) { W[i] = x; });
    if (S != Sin) each((int)p.P, [&](int i) { return Sin[i]; }, [&](int i, float x) { S[i] = x; });
  }
  __syncthreads();
  if (p.N == 0) return;
  float* const wsb = (in_lds ? dyn_lds + 2 * p.P4 : p.ws + (int64_t)s * p.ws_stride) + (one ? (int64_t)(cs & 1) * p.region : 0);
  const WsLayout& lay = p.lay;
  struct {
    float *vin, *sc, *D, *A, *E, *F, *U;
  } w = {wsb + lay.vin, wsb + lay.sc, wsb + lay.D, wsb + lay.A, wsb + lay.E, wsb + lay.F, wsb + lay.U};
  auto act = [&](int l) { return wsb + lay.act[l]; };
  auto spv = [&](int l) { return wsb + lay.sp[l]; };
  auto delta = [&](int l) { return wsb + lay.delta[l]; };
  auto hq = [&](int i) { return wsb + lay.hq[i]; };
  const int64_t tok0 = (int64_t)s * p.N;
  const bool all = stage == kAllStages;
  auto run = [&](int st, int l) { return all || (stage == st && layer == l); };

  for (int c0 = one ? cs * p.chunk : 0; c0 < p.N; c0 += p.chunk) {
    const int n = min(p.chunk, p.N - c0);
    if (p.ckpt) {
      // the state at this chunk's start (read only here; it is next written
      // by this chunk's fold, many barriers later)
      float* ck = p.ckpt + (int64_t)s * p.ckpt_stride + (int64_t)(c0 / p.chunk) * 2 * p.P;
      each(
          (int)p.P, [&](int i) { return make_float2(Wr[i], Sr[i]); },
          [&](int i, float2 x) {
            ck[i] = x.x;
            ck[p.P + i] = x.y;
          });
      // a sweep for checkpoints only ends at the last chunk's start
      if (!p.y && c0 + p.chunk >= p.N) break;
    }
    // the chunk's gates: token j at index j * gs (one shared value when the
    // gates are given per chunk)
    const int64_t g0 = p.chunk_gates ? (int64_t)s * ((p.N + p.chunk - 1) / p.chunk) + c0 / p.chunk : tok0 + c0;
    const int gs = p.chunk_gates ? 0 : 1;
    const float* al = p.alpha + g0;
    const float* et = p.eta + g0;
    const float* th = p.theta + g0;

    // ---- load the chunk's keys, values and queries (fp32 copies) ----
    if (all || stage == kLoad) {
      float* a0 = act(0);
      float* q0 = hq(0);
      each(
          n * d,
          [&](int e) {
            const int64_t gi = (tok0 + c0) * d + e;
            return make_float3(sweep ? load_io(p.k, gi, p.io) : 0.f, sweep ? load_io(p.v, gi, p.io) : 0.f,
                               rd ? load_io(p.q, gi, p.io) : 0.f);
          },
          [&](int e, float3 x) {
            if (sweep) {
              a0[e] = x.x;
              w.vin[e] = x.y;
            }
            if (rd) q0[(e / d) * p.maxw + (e % d)] = x.z;
          });
    }
    // ---- a1: coefficient recurrences (one thread per column i of D) ----
    // (gates read kBatch steps ahead of the stores, which may alias them)
    const bool coef = sweep && (all || stage == kLoad);
    for (int i = tid; i < n && coef; i += kThreads) {
      const float ti = th[i * gs];
      float di = ti, pr = 1.f;
      for (int j = 0; j < i; ++j) w.D[j * n + i] = 0.f;
      w.D[i * n + i] = di;
      for (int j0 = i + 1; j0 < n; j0 += kBatch) {
        float ev[kBatch], av[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = min(j0 + u, n - 1);
          ev[u] = et[j * gs];
          av[u] = al[j * gs];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (j0 + u < n) {
            pr *= ev[u];
            di = (1.f - av[u]) * di + ti * pr;
            w.D[(j0 + u) * n + i] = di;
          }
        }
      }
      w.U[i] = ti * pr;
    }
    // A, E, F on the last thread, whose columns above are the shortest, so
    // its recurrence runs beside the long ones of the first wave
    if (tid == kThreads - 1 && coef) {
      float a = 1.f, e = 1.f, f = 0.f;
      for (int j0 = 0; j0 < n; j0 += kBatch) {
        float ev[kBatch], av[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = min(j0 + u, n - 1);
          ev[u] = et[j * gs];
          av[u] = al[j * gs];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (j0 + u < n) {
            a *= 1.f - av[u];
            e *= ev[u];
            f = (1.f - av[u]) * f + e;
            w.A[j0 + u] = a;
            w.E[j0 + u] = e;
            w.F[j0 + u] = f;
          }
        }
      }
    }
    __syncthreads();

    // ---- a2: key-side forward at the chunk-start weights ----
    for (int l = 1; l <= L && sweep; ++l) {
      if (!run(kKey, l)) continue;
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = Wr + p.off[l];
      const float* ain = act(l - 1);
      float* aout = act(l);
      float* spl = spv(l);
      float* dl = delta(l);
      const float* vin = w.vin;
      const bool last = (l == L);
      block_gemm<true>(
          n, nout, nin, [=](int j, int c) { return ain[j * nin + c]; },
          [=](int c, int r) { return Wl[(int64_t)r * nin + c]; }, kB_KMAJOR,
          [=](int j, int r) { return last ? vin[j * nout + r] : 0.f; },
          [=](int j, int r, float z, float vv, bool ok) {
            if (last) {
              if (ok) {
                aout[j * nout + r] = z;
                dl[j * nout + r] = z - vv;  // a3: residual M(k) - v
              }
            } else if (ok) {
              aout[j * nout + r] = silu(z);
              spl[j * nout + r] = silu_prime(z);
            }
          });
    }
    // ---- a3: backprop to every layer's delta ----
    for (int l = L; l >= 2 && sweep; --l) {
      if (!run(kBack, l)) continue;
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = Wr + p.off[l];
      const float* dl = delta(l);
      float* dprev = delta(l - 1);
      const float* spp = spv(l - 1);
      block_gemm<true>(
          n, nin, nout, [=](int j, int r) { return dl[j * nout + r]; },
          [=](int r, int c) { return Wl[(int64_t)r * nin + c]; }, kB_NMAJOR,
          [=](int j, int c) { return spp[j * nin + c]; },
          [=](int j, int c, float x, float sp, bool ok) {
            if (ok) dprev[j * nin + c] = x * sp;
          });
    }
    // ---- a5: retrieval ----
    for (int l = 1; l <= L && rd; ++l) {
      if (!run(kScores, l) && !run(kRead, l)) continue;
      const int cur = (l - 1) & 1;   // query-side activations ping-pong
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = Wr + p.off[l];
      const float* Sl = Sr + p.off[l];
      const float* h = hq(cur);
      float* hn = hq(cur ^ 1);
      const float* ak = act(l - 1);
      const float* dl = delta(l);
      const bool last = (l == L);
      const int maxw = p.maxw;
      auto epi = [=](int j, int r, float zq, bool ok) {
        if (!ok) return;
        if (last)
          store_io(p.y, (tok0 + c0 + j) * d + r, zq, p.io);
        else
          hn[j * maxw + r] = silu(zq);
      };
      if (p.read_mode == TM_READ_CHUNK_START) {
        if (run(kRead, l))
          block_gemm<true>(
              n, nout, nin, [=](int j, int c) { return h[j * maxw + c]; },
              [=](int c, int r) { return Wl[(int64_t)r * nin + c]; }, kB_KMAJOR, epi);
      } else {
        float* sc = w.sc;
        const float* D = w.D;
        // masked, decay-weighted scores (D o (h a^T)), lower triangle
        if (run(kScores, l))
        block_gemm<true>(
            n, n, nin, [=](int j, int c) { return h[j * maxw + c]; },
            [=](int c, int i) { return ak[i * nin + c]; }, kB_KMAJOR,
            [=](int j, int i) { return D[j * n + i]; },
            [=](int j, int i, float x, float dji, bool ok) {
              if (ok) sc[j * n + i] = (i <= j) ? dji * x : 0.f;
            });
        const float* A = w.A;
        const float* F = w.F;
        // zq = diag(A) h W^T + diag(F) h S^T - sc delta, as one contraction
        // over the concatenated index [W-part | S-part | token part]
        if (run(kRead, l))
        block_gemm<true>(
            n, nout, 2 * nin + n,
            [=](int j, int kk) {   // branch-free: pick the address, then the factor
              const bool st = kk < 2 * nin;   // every arm's offset kept in range (only one is read)
              const int kc = kk < nin ? kk : (st ? kk - nin : 0), kt = st ? 0 : kk - 2 * nin;
              const float* x = st ? h + j * maxw + kc : sc + j * n + kt;
              const float f = *(kk < nin ? A + j : F + j);
              const float v = *x;
              return st ? f * v : -v;
            },
            [=](int kk, int r) {
              const int kw = kk < nin ? kk : 0, ks = kk >= nin && kk < 2 * nin ? kk - nin : 0,
                        kt = kk >= 2 * nin ? kk - 2 * nin : 0;
              const float* x = kk < nin       ? Wl + (int64_t)r * nin + kw
                               : kk < 2 * nin ? Sl + (int64_t)r * nin + ks
                                              : dl + (int64_t)kt * nout + r;
              return *x;
            },
            [=](int k0) { return k0 + kGk <= 2 * nin; },   // the token part is contiguous in r
            epi);
      }
    }
    // ---- a4: fold the chunk into the state (after every read of W_0, S_0) ----
    if (sweep) {
      const float An = w.A[n - 1], En = w.E[n - 1], Fn = w.F[n - 1];
      const float* Dlast = w.D + (n - 1) * n;
      const float* U = w.U;
      for (int l = 1; l <= L; ++l) {
        const int nin = p.widths[l - 1], nout = p.widths[l];
        const float* Wl = Wr + p.off[l];
        const float* Sl = Sr + p.off[l];
        float* Wo = W + p.off[l];
        float* So = S + p.off[l];
        const float* dl = delta(l);
        const float* ak = act(l - 1);
        if (run(kFoldW, l))
        block_gemm<false>(
            nout, nin, n, [=](int r, int j) { return Dlast[j] * dl[j * nout + r]; },
            [=](int j, int c) { return ak[j * nin + c]; }, kB_NMAJOR,
            [=](int r, int c) {
              const int64_t i = (int64_t)r * nin + c;
              return An * Wl[i] + Fn * Sl[i];
            },
            [=](int r, int c, float g, float base, bool ok) {
              if (ok) Wo[(int64_t)r * nin + c] = base - g;
            });
        if (run(kFoldS, l))
        block_gemm<false>(
            nout, nin, n, [=](int r, int j) { return U[j] * dl[j * nout + r]; },
            [=](int j, int c) { return ak[j * nin + c]; }, kB_NMAJOR,
            [=](int r, int c) { return En * Sl[(int64_t)r * nin + c]; },
            [=](int r, int c, float g, float base, bool ok) {
              if (ok) So[(int64_t)r * nin + c] = base - g;
            });
      }
    }
    __syncthreads();
    if (one) break;
  }
  if (in_lds) {   // the final state back to global memory
    each((int)p.P, [&](int i) { return W[i]; }, [&](int i, float x) { Wg[i] = x; });
    each((int)p.P, [&](int i) { return S[i]; }, [&](int i, float x) { Sg[i] = x; });
  }
}

// y = M_W(q) for a tile of tokens; activations ping-pong through LDS.
__global__ void __launch_bounds__(kThreads) retrieve_kernel(GParams p) {
  __shared__ float buf[2][kRetrieveTile * kMaxWidthRetrieve];
  const int s = blockIdx.y;
  const int t0 = blockIdx.x * kRetrieveTile;
  const int n = min(kRetrieveTile, p.N - t0);
  const int tid = threadIdx.x;
  const int d = p.d;
  const int64_t tok0 = (int64_t)s * p.N + t0;
  const float* W = p.W_in + (int64_t)s * p.P;
  // kRetrieveTile rows of stride maxw (<= kMaxWidthRetrieve) per buffer
  float* h = buf[0];
  float* hn = buf[1];
  const int stride = p.maxw;
  for (int e = tid; e < n * d; e += kThreads) h[(e / d) * stride + e % d] = load_io(p.q, tok0 * d + e, p.io);
  __syncthreads();
  for (int l = 1; l <= p.L; ++l) {
    const int nin = p.widths[l - 1], nout = p.widths[l];
    const float* Wl = W + p.off[l];
    const bool last = (l == p.L);
    for (int e = tid; e < n * nout; e += kThreads) {
      const int j = e / nout, r = e % nout;
      const float* wr = Wl + (int64_t)r * nin;
      const float* hr = h + j * stride;
      float acc = 0.f;
      for (int c = 0; c < nin; ++c) acc = fmaf(wr[c], hr[c], acc);
      if (last)
        store_io(p.y, (tok0 + j) * d + r, acc, p.io);
      else
        hn[j * stride + r] = silu(acc);
    }
    __syncthreads();
    float* t = h;
    h = hn;
    hn = t;
  }
}

// LDS mode when the state and the workspace fit the budget; returns the
// dynamic LDS bytes of the launch (0: global memory)
int set_lds_mode(GParams& p) {
  p.P4 = (p.P + 3) / 4 * 4;
  const int64_t bytes = (2 * p.P4 + p.lay.total) * (int64_t)sizeof(float);
  p.lds_state = p.N > 0 && bytes <= kLdsStateBytes;
  return p.lds_state ? (int)bytes : 0;
}

hipError_t launch_generic_kernel(const GParams& p, int streams, int lds, hipStream_t stream, int cs = -1,
                                 int phase = kBoth, int stage = kAllStages, int layer = 0, int ytiles = 1) {
  if (lds > 0) {
    const hipError_t e = hipFuncSetAttribute((const void*)generic_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(generic_kernel, dim3(streams, ytiles), dim3(kThreads), lds, stream, p, cs, phase, stage, layer);
  return hipGetLastError();
}

// output tiles of an M x N block_gemm contraction
int gemm_tiles(int M, int N) {
  const int tn = N > kGemmTile ? kGN : kGemmTile;
  return ((M + kGemmTile - 1) / kGemmTile) * ((N + tn - 1) / tn);
}

int rows_reserved(const Shape& s, int chunk) { return chunk < s.N ? chunk : (s.N > 0 ? s.N : 1); }

// LDS mode (set_lds_mode) for this shape and chunk
bool lds_fits(const Shape& s, int b) {
  return s.N > 0 && (2 * ((s.P + 3) / 4 * 4) + ws_layout(s, b).total) * (int64_t)sizeof(float) <= kLdsStateBytes;
}

// The forward call runs one chunk per launch, sweep and reads side by side,
// when the state is too large for LDS (so the per-chunk work is large) and
// the chunks are long enough for the per-launch cost not to matter.
bool split_forward(const Shape& s, int chunk) {
  return !lds_fits(s, rows_reserved(s, chunk)) && chunk >= 16 && s.N > chunk;
}

GParams make_params(const Shape& s, int chunk) {
  GParams p{};
  p.N = s.N;
  p.d = s.d;
  p.L = s.L;
  p.io = s.io;
  p.read_mode = s.read_mode;
  p.chunk_gates = s.chunk_gates;
  p.chunk = chunk;
  for (int l = 0; l <= s.L; ++l) p.widths[l] = s.widths[l];
  for (int l = 1; l <= s.L; ++l) p.off[l] = s.off[l];
  p.P = s.P;
  p.maxw = s.maxw;
  return p;
}

}  // namespace

int64_t generic_ws_floats_per_stream(const Shape& s, int b) { return ws_layout(s, b).total; }

int64_t generic_forward_ws_floats_per_stream(const Shape& s, int chunk) {
  const int64_t region = ws_layout(s, rows_reserved(s, chunk)).total;   // a multiple of 64
  if (!split_forward(s, chunk)) return region;
  return 2 * region + 4 * ((s.P + 63) / 64 * 64);   // two regions, two rotating (W, S) buffers
}

hipError_t launch_generic(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                          const float* alpha, const float* eta, const float* theta,
                          const float* W_in, const float* S_in, void* y, float* W_out,
                          float* S_out, float* ws, hipStream_t stream) {
  if (linear_supported(s, chunk))
    return launch_linear(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, y, W_out, S_out, stream);
  GParams p = make_params(s, chunk);
  p.b = rows_reserved(s, chunk);
  p.lay = ws_layout(s, p.b);
  p.k = k;
  p.v = v;
  p.q = q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.W_in = W_in;
  p.S_in = S_in;
  p.in_stride = s.P;
  p.y = y;
  p.W = W_out;
  p.S = S_out;
  p.state_stride = s.P;
  p.ckpt = nullptr;
  p.ckpt_stride = 0;
  p.ws = ws;
  p.ws_stride = generic_forward_ws_floats_per_stream(s, chunk);
  // (an in-place call keeps the single launch: chunk 0's reads need the
  // input state after the output buffers have started to rotate)
  if (!split_forward(s, chunk) || W_out == W_in || S_out == S_in)
    return launch_generic_kernel(p, s.streams, set_lds_mode(p), stream);

  // One chunk per launch.  Chunk c's start state is buffer c % 3 (c = 0: the
  // inputs) and its fold goes to buffer (c + 1) % 3; buffer nchunks % 3 is
  // (W_out, S_out), the other two follow the regions in the workspace.  The
  // sweep of chunk c waits for the reads of chunk c - 2, which used its
  // region and its destination buffer; the reads of chunk c wait for its sweep.
  p.region = p.lay.total;
  const int nchunks = (s.N + chunk - 1) / chunk;
  const int64_t pb = (s.P + 63) / 64 * 64;
  float* wsbuf = ws + 2 * p.region;
  struct Buf { float *W, *S; int64_t stride; } buf[3];
  for (int i = 0, j = 0; i < 3; ++i) {
    if (i == nchunks % 3) {
      buf[i] = Buf{W_out, S_out, s.P};
    } else {
      buf[i] = Buf{wsbuf + 2 * pb * j, wsbuf + 2 * pb * j + pb, p.ws_stride};
      ++j;
    }
  }
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return err;
  // with at least half the CUs idle under one workgroup per stream and
  // phase, every step gets a launch of its own and its contraction's tiles
  // spread over workgroups; otherwise one launch per phase (short launches
  // would then cost more than they spread)
  const bool per_step = 4 * (int64_t)s.streams <= cus;
  std::unique_lock<std::mutex> lock;
  SideStream* x = nullptr;
  if ((err = side_stream(dev, &x, lock)) != hipSuccess) return err;
  auto chunks = [&]() -> hipError_t {
    hipError_t e;
    for (int c = 0; c < nchunks; ++c) {
      const Buf src = c == 0 ? Buf{(float*)W_in, (float*)S_in, s.P} : buf[c % 3], dst = buf[(c + 1) % 3];
      p.W_in = src.W;
      p.S_in = src.S;
      p.in_stride = src.stride;
      p.W = dst.W;
      p.S = dst.S;
      p.state_stride = dst.stride;
      // per step: one launch per step, each contraction's output tiles shared
      // out over the workgroups of the launch's y dimension
      const int n = std::min(chunk, s.N - c * chunk);
      auto step = [&](hipStream_t st, int phase, int stage, int l, int M, int N) {
        return launch_generic_kernel(p, s.streams, 0, st, c, phase, stage, l, gemm_tiles(M, N));
      };
      const int* wd = s.widths;
      if (c >= 2 && (e = hipStreamWaitEvent(stream, x->cons[c & 1], 0)) != hipSuccess) return e;
      if (!per_step) {
        if ((e = launch_generic_kernel(p, s.streams, 0, stream, c, kSweep)) != hipSuccess) return e;
        if ((e = hipEventRecord(x->prod[c & 1], stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(x->st, x->prod[c & 1], 0)) != hipSuccess) return e;
        if ((e = launch_generic_kernel(p, s.streams, 0, x->st, c, kReads)) != hipSuccess) return e;
        if ((e = hipEventRecord(x->cons[c & 1], x->st)) != hipSuccess) return e;
        continue;
      }
      if ((e = step(stream, kSweep, kLoad, 0, 1, 1)) != hipSuccess) return e;
      for (int l = 1; l <= s.L; ++l)
        if ((e = step(stream, kSweep, kKey, l, n, wd[l])) != hipSuccess) return e;
      for (int l = s.L; l >= 2; --l)
        if ((e = step(stream, kSweep, kBack, l, n, wd[l - 1])) != hipSuccess) return e;
      for (int l = 1; l <= s.L; ++l) {
        if ((e = step(stream, kSweep, kFoldW, l, wd[l], wd[l - 1])) != hipSuccess) return e;
        if ((e = step(stream, kSweep, kFoldS, l, wd[l], wd[l - 1])) != hipSuccess) return e;
      }
      if ((e = hipEventRecord(x->prod[c & 1], stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(x->st, x->prod[c & 1], 0)) != hipSuccess) return e;
      if ((e = step(x->st, kReads, kLoad, 0, 1, 1)) != hipSuccess) return e;
      for (int l = 1; l <= s.L; ++l) {
        if (s.read_mode != TM_READ_CHUNK_START && (e = step(x->st, kReads, kScores, l, n, n)) != hipSuccess) return e;
        if ((e = step(x->st, kReads, kRead, l, n, wd[l])) != hipSuccess) return e;
      }
      if ((e = hipEventRecord(x->cons[c & 1], x->st)) != hipSuccess) return e;
    }
    return hipSuccess;
  };
  // the side stream's last work is the reads of the last chunk: the join
  // makes the caller's stream wait for it (and for whatever was enqueued
  // before an error)
  return join_side(x, stream, chunks());
}

hipError_t launch_generic_checkpoints(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                                      const float* alpha, const float* eta, const float* theta, const float* W_in,
                                      const float* S_in, float* W, float* S, int64_t state_stride, float* ckpt,
                                      int64_t ckpt_stride, float* ws, int64_t ws_stride, hipStream_t stream) {
  GParams p = make_params(s, chunk);
  p.b = chunk < s.N ? chunk : (s.N > 0 ? s.N : 1);
  p.lay = ws_layout(s, p.b);
  p.k = k;
  p.v = v;
  p.q = q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.W_in = W_in;
  p.S_in = S_in;
  p.in_stride = s.P;
  p.y = nullptr;
  p.W = W;
  p.S = S;
  p.state_stride = state_stride;
  p.ckpt = ckpt;
  p.ckpt_stride = ckpt_stride;
  p.ws = ws;
  p.ws_stride = ws_stride;
  return launch_generic_kernel(p, s.streams, set_lds_mode(p), stream);
}

hipError_t launch_retrieve_generic(const Shape& s, const void* q, const float* W, void* y,
                                   hipStream_t stream) {
  GParams p = make_params(s, 1);
  p.q = q;
  p.W_in = W;
  p.y = y;
  dim3 grid((s.N + kRetrieveTile - 1) / kRetrieveTile, s.streams);
  hipLaunchKernelGGL(retrieve_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace titans
