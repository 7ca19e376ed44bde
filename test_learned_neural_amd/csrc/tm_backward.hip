// Backward pass through the memory: gradients of a loss with respect to
// every input of titans_mem_forward (k, v, q, the gates, W_in, S_in), for
// the outer loop that trains whatever produces those inputs ("Titans:
// Learning to Memorize at Test Time", mer.dev notes, section 3.1
// "Objective": the memory's parameters are the inner loop, the rest of the
// architecture the outer one).
//
// Forward being differentiated, chunk by chunk (section 3.2: every gradient
// of a chunk is taken at its chunk-start weights W; momentum and forgetting
// of section 3.1).  Per layer, with g_i = delta_i a_i^T the inner gradient
// of token i at W, and the chunk coefficients of the gates (t, i local):
//   A_t = prod_{m<=t} (1 - alpha_m)   E_t = prod_{m<=t} eta_m
//   F_t = (1 - alpha_t) F_{t-1} + E_t  P[t,i] = prod_{i<m<=t} eta_m
//   D[t,i] = (1 - alpha_t) D[t-1,i] + theta_i P[t,i]  (D[i,i] = theta_i)
//   U_i = theta_i P[n-1,i]
// the state after token t is W_t = A_t W + F_t S - sum_{i<=t} D[t,i] g_i,
// the chunk ends at (W_{n-1}, E_{n-1} S - sum_i U_i g_i), and the read of
// token t (after its write) is, layer by layer from h^0 = q_t,
//   zq^l_t = A_t W h_t + F_t S h_t - sum_{i<=t} D[t,i] (a_i . h_t) delta_i.
//
// Reverse mode runs over the chunks from the last, carrying the adjoints
// (Wbar, Sbar) of the chunk-end state.  Per chunk, from the chunk-start
// checkpoint (W, S), every step is a contraction over the chunk's tokens or
// over a layer width, i.e. a matrix product of the same shapes as the
// forward's closed form (adjoints carry a bar; rho^l_t = dL/dzq^l_t):
//   reads    rho^L = dy;  Abar_t += rho.(W h), Fbar_t += rho.(S h)
//            Dbar[t,i] -= (rho_t . delta_i)(a_i . h_t)
//            hbar = A W^T rho + F S^T rho - sum_i D[t,i] (rho_t . delta_i) a_i
//            rho^{l-1} = hbar * SiLU'(zq^{l-1}),  qbar = hbar at l = 1
//            deltabar_i -= sum_t D[t,i] (a_i . h_t) rho_t
//            abar_i     -= sum_t D[t,i] (rho_t . delta_i) h_t
//   fold     deltabar_i -= D[n-1,i] Wbar a_i + U_i Sbar a_i
//            abar_i     -= D[n-1,i] Wbar^T delta_i + U_i Sbar^T delta_i
//            Dbar[n-1,i] -= delta_i . Wbar a_i,  Ubar_i -= delta_i . Sbar a_i
//            Abar_{n-1} += <Wbar, W>, Fbar_{n-1} += <Wbar, S>, Ebar_{n-1} = <Sbar, S>
//   inner gradient (delta^L = a^L - v, delta^l = b^l * SiLU'(z^l) with
//            b^l = W^{l+1 T} delta^{l+1}; its backward pass carries the
//            second-order terms):
//            bbar^l = deltabar^l * SiLU'(z^l), zbar^l = deltabar^l * b^l * SiLU''(z^l),
//            deltabar^{l+1} += W^{l+1} bbar^l;  vbar = -deltabar^L, zbar^L = deltabar^L;
//            zbar^l += abar^l * SiLU'(z^l), abar^{l-1} += W^{l T} zbar^l;  kbar = abar^0
//   state    Sbar <- F_{n-1} Wbar + E_{n-1} Sbar + sum_t F_t rho_t h_t^T
//            Wbar <- A_{n-1} Wbar + sum_t A_t rho_t h_t^T
//                    + sum_i (delta^l_i bbar^{l-1 T}_i + zbar^l_i a^{l-1 T}_i)
//   gates    the adjoints of A, E, F, D, P, U back through their recurrences
// With the chunk-start read, zq^l_t = W h_t: hbar = W^T rho and Wbar gains
// sum_t rho_t h_t^T; no coefficient enters the reads.
//
// Execution: a forward sweep (the generic kernel's chunked closed form,
// without retrieval) stores (W, S) at every chunk start in the workspace;
// then the chunks are walked backwards, one workgroup per stream and two
// launches per chunk: the part of a chunk that does not depend on the
// carried adjoints (inputs, coefficients, key side, reads) runs on a second
// stream one chunk ahead of the rest, so the two overlap on the device.
// Every product is block_gemm (fp32 on the matrix cores); a chunk's vectors
// live in one of two per-stream workspace regions (chunk parity), the
// adjoints (Wbar, Sbar) in dW_in, dS_in.
#include "tm_internal.h"
#include "tm_block_gemm.h"

#include <hip/hip_bf16.h>

#include <algorithm>
#include <mutex>

namespace titans {
namespace {

constexpr int kBT = kGemmThreads;   // threads per workgroup
constexpr int kBW = kBT / 64;

// Per-stream workspace region of the reverse sweep (float offsets, b rows
// per chunk; "[b x n_l]" is token-major).  Filled on the host.
struct BwLayout {
  int64_t act[kMaxLayers + 1];   // a^l of the keys, l = 0..L (a^0 = k)       [b x n_l]
  int64_t z[kMaxLayers + 1];     // z^l, l = 1..L-1
  int64_t dl[kMaxLayers + 1];    // delta^l, l = 1..L
  int64_t bv[kMaxLayers + 1];    // b^l = W^{l+1 T} delta^{l+1}, l = 1..L-1
  int64_t h[kMaxLayers + 1];     // read activations h^l, l = 0..L-1 (h^0 = q)
  int64_t zq[kMaxLayers + 1];    // read pre-activations, l = 1..L-1
  int64_t uw[kMaxLayers + 1];    // W^l h^{l-1}, l = 1..L
  int64_t us[kMaxLayers + 1];    // S^l h^{l-1}, l = 1..L
  int64_t rho[kMaxLayers + 1];   // dL/dzq^l, l = 1..L
  int64_t sc[kMaxLayers + 1];    // a^{l-1}_i . h^{l-1}_t, l = 1..L           [b x b], [t][i]
  int64_t dbar[kMaxLayers + 1];  // deltabar^l, l = 1..L (also zbar^L)
  int64_t abar[kMaxLayers + 1];  // abar^l, l = 0..L-1
  int64_t bbar[kMaxLayers + 1];  // bbar^l, l = 1..L-1
  int64_t zbar[kMaxLayers + 1];  // zbar^l, l = 1..L-1
  int64_t vin, xw, xs;           // v [b x d]; Wbar a, Sbar a [b x maxw]
  int64_t dsc, dr;               // -D o sc, -D o (rho delta^T)               [b x b]
  int64_t D, P, Dbar, Ca, Ce;    // [b x b]
  int64_t A, E, F, U, Abar, Fbar, Ubar, ga, ge, gt;   // [b]
  int64_t red;                   // 64 floats
  int64_t total;
};

struct BwdParams {
  int N, chunk, nchunks, b, L, d, io, read_mode, chunk_gates;
  int w[kMaxLayers + 1];
  int64_t off[kMaxLayers + 1];
  int64_t P;
  int maxw;
  const void* k;
  const void* v;
  const void* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  const float* dy;
  const float* dW_out;
  const float* dS_out;
  float* dk;
  float* dv;
  float* dq;
  float* dalpha;
  float* deta;
  float* dtheta;
  float* dW_in;       // Wbar during the sweep
  float* dS_in;       // Sbar during the sweep
  float* ws;
  int64_t ws_stream;  // floats per stream
  int64_t o_buf;      // offset of the reverse sweep's two regions (checkpoints before them)
  int64_t region;     // floats per region
  BwLayout lay;
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror: every lane holds its 16-lane group's sum
  return __shfl(x, 0) + __shfl(x, 16) + __shfl(x, 32) + __shfl(x, 48);
}
// total over the workgroup, returned to every thread
__device__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kBW; ++i) t += red[i];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float sgm(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float silu(float z) { return z * sgm(z); }
__device__ __forceinline__ float dsilu(float z) { const float s = sgm(z); return s * (1.f + z * (1.f - s)); }
__device__ __forceinline__ float d2silu(float z) {
  const float s = sgm(z);
  return s * (1.f - s) * (2.f + z * (1.f - 2.f * s));
}

__device__ __forceinline__ float io_load(const void* base, int io, int64_t i) {
  if (io == TM_IO_BF16) return __bfloat162float(((const __hip_bfloat16*)base)[i]);
  return ((const float*)base)[i];
}

// out[t] += scale * sum_{c < w} X[t*ldx + c] * Y[t*ldy + c] for rows t < n,
// one wave per row; the row sums of a round of kBT rows stay in lanes (row
// t0 + wave + kBW j in lane j) and are stored once at the round's end.  No
// barrier inside.
__device__ void row_dots(float* out, const float* X, int ldx, const float* Y, int ldy, int n, int w,
                         float scale = 1.f) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t0 = 0; t0 < n; t0 += kBT) {
    const int jn = min(64, (n - t0 - wv + kBW - 1) / kBW);   // this wave's rows in the round
    float held = 0.f;
    for (int j0 = 0; j0 < jn; j0 += 4) {                     // four rows' loads in flight together
      int64_t ox[4], oy[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = t0 + wv + kBW * min(j0 + u, jn - 1);
        ox[u] = t * ldx;
        oy[u] = t * ldy;
      }
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c = lane; c < w; c += 64) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += X[ox[u] + c] * Y[oy[u] + c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float r = wave_sum(acc[u]);
        held = lane == j0 + u ? r : held;   // lanes past the wave's rows are never stored
      }
    }
    const int t = t0 + wv + kBW * lane;
    if (t < n) out[t] += scale * held;
  }
}

// One chunk c of the reverse sweep, one workgroup per stream, in two phases
// launched separately: kProduce (the chunk's inputs, coefficients, key side
// and the reads -- nothing that depends on the carried adjoints) and
// kConsume (the fold, the inner gradient's backward, the state adjoints and
// the gates).  Chunk c's phase-1 results sit in workspace region c % 2, so
// phase 1 of chunk c - 1 can run beside phase 2 of chunk c.
enum { kProduce = 1, kConsume = 2 };

__global__ void __launch_bounds__(kBT) backward_kernel(BwdParams p, int c, int phase) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = p.L, d = p.d, bb = p.b, mw = p.maxw;
  const int64_t P = p.P;
  float* const Wb = p.dW_in + (int64_t)s * P;
  float* const Sb = p.dS_in + (int64_t)s * P;
  if (phase == kConsume && c == p.nchunks - 1) {
    each(
        (int)P,
        [&](int i) {
          return make_float2(p.dW_out ? p.dW_out[(int64_t)s * P + i] : 0.f, p.dS_out ? p.dS_out[(int64_t)s * P + i] : 0.f);
        },
        [&](int i, float2 x) {
          Wb[i] = x.x;
          Sb[i] = x.y;
        });
    __syncthreads();
  }
  float* const base = p.ws + (int64_t)s * p.ws_stream;
  float* const wsb = base + p.o_buf + (int64_t)(c & 1) * p.region;
  const BwLayout& y = p.lay;
  auto V = [&](int64_t o) { return wsb + o; };
  float* const red = V(y.red);
  float* const cA = V(y.A);
  float* const cE = V(y.E);
  float* const cF = V(y.F);
  float* const cU = V(y.U);
  float* const cD = V(y.D);
  float* const cP = V(y.P);
  float* const Abar = V(y.Abar);
  float* const Fbar = V(y.Fbar);
  float* const Ubar = V(y.Ubar);
  float* const Dbar = V(y.Dbar);
  float* const Ca = V(y.Ca);
  float* const Ce = V(y.Ce);
  float* const ga = V(y.ga);
  float* const ge = V(y.ge);
  float* const gt = V(y.gt);
  float* const vin = V(y.vin);
  float* const xw = V(y.xw);
  float* const xs = V(y.xs);
  float* const dsc = V(y.dsc);
  float* const dr = V(y.dr);
  const bool reads = p.dy != nullptr;
  const bool cstart = p.read_mode == TM_READ_CHUNK_START;
  const int64_t tok0 = (int64_t)s * p.N;
  const int c0 = c * p.chunk;
  const int n = min(p.chunk, p.N - c0);
  const float* const W = base + (int64_t)c * 2 * P;   // chunk-start checkpoint
  const float* const S = W + P;
  const int64_t g0 = p.chunk_gates ? (int64_t)s * p.nchunks + c : tok0 + c0;
  const int gs = p.chunk_gates ? 0 : 1;
  const float* al = p.alpha + g0;
  const float* et = p.eta + g0;
  const float* th = p.theta + g0;
  const int64_t row0 = tok0 + c0;                     // first token row of the chunk

  if (phase == kProduce) {
    // ---- chunk inputs; adjoint accumulators cleared ----
    {
      float* a0 = V(y.act[0]);
      float* h0 = V(y.h[0]);
      float* rL = V(y.rho[L]);
      each(
          n * d,
          [&](int e) {
            const int64_t gi = row0 * d + e;
            return make_float4(io_load(p.k, p.io, gi), io_load(p.v, p.io, gi), reads ? io_load(p.q, p.io, gi) : 0.f,
                               reads ? p.dy[gi] : 0.f);
          },
          [&](int e, float4 x) {
            a0[e] = x.x;
            vin[e] = x.y;
            if (reads) {
              h0[e] = x.z;
              rL[e] = x.w;
            } else {
              p.dq[row0 * d + e] = 0.f;
            }
          });
    }
    for (int l = 0; l <= L; ++l) {
      if (l >= 1)
        for (int e = tid; e < n * p.w[l]; e += kBT) V(y.dbar[l])[e] = 0.f;
      if (l < L)
        for (int e = tid; e < n * p.w[l]; e += kBT) V(y.abar[l])[e] = 0.f;
    }
    for (int e = tid; e < n * bb; e += kBT) Dbar[e] = 0.f;
    for (int e = tid; e < n; e += kBT) {
      Abar[e] = 0.f;
      Fbar[e] = 0.f;
      Ubar[e] = 0.f;
    }
    // ---- coefficients: one thread per column i of D and P ----
    for (int i = tid; i < n; i += kBT) {
      const float ti = th[i * gs];
      float di = ti, pr = 1.f;
      for (int t = 0; t < i; ++t) {
        cD[t * bb + i] = 0.f;
        cP[t * bb + i] = 0.f;
      }
      cD[i * bb + i] = di;
      cP[i * bb + i] = 1.f;
      for (int t0 = i + 1; t0 < n; t0 += kBatch) {
        float ev[kBatch], av[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = min(t0 + j, n - 1);
          ev[j] = et[t * gs];
          av[j] = al[t * gs];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (t0 + j < n) {
            pr *= ev[j];
            di = (1.f - av[j]) * di + ti * pr;
            cD[(t0 + j) * bb + i] = di;
            cP[(t0 + j) * bb + i] = pr;
          }
        }
      }
      cU[i] = ti * pr;
    }
    // A, E, F on the last thread, whose columns above are the shortest, so
    // its recurrence runs beside the long ones of the first wave
    if (tid == kBT - 1) {
      float a = 1.f, e = 1.f, f = 0.f;
      for (int t0 = 0; t0 < n; t0 += kBatch) {
        float ev[kBatch], av[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = min(t0 + j, n - 1);
          ev[j] = et[t * gs];
          av[j] = al[t * gs];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (t0 + j < n) {
            a *= 1.f - av[j];
            e *= ev[j];
            f = (1.f - av[j]) * f + e;
            cA[t0 + j] = a;
            cE[t0 + j] = e;
            cF[t0 + j] = f;
          }
        }
      }
    }
    __syncthreads();

    // ---- key side at W: z^l, a^l, delta^l, b^l ----
    for (int l = 1; l <= L; ++l) {
      const int nin = p.w[l - 1], nout = p.w[l];
      const float* Wl = W + p.off[l];
      const float* ain = V(y.act[l - 1]);
      float* aout = V(y.act[l]);
      float* zl = V(y.z[l]);
      float* dl = V(y.dl[l]);
      const bool last = l == L;
      block_gemm<true>(
          n, nout, nin, [=](int j, int cc) { return ain[j * nin + cc]; },
          [=](int cc, int r) { return Wl[(int64_t)r * nin + cc]; }, kB_KMAJOR,
          [=](int j, int r) { return last ? vin[j * nout + r] : 0.f; },
          [=](int j, int r, float x, float vv, bool ok) {
            if (last) {
              if (ok) {
                aout[j * nout + r] = x;
                dl[j * nout + r] = x - vv;
              }
            } else if (ok) {
              zl[j * nout + r] = x;
              aout[j * nout + r] = silu(x);
            }
          });
    }
    for (int l = L - 1; l >= 1; --l) {
      const int nl = p.w[l], nu = p.w[l + 1];
      const float* Wu = W + p.off[l + 1];
      const float* du = V(y.dl[l + 1]);
      const float* zl = V(y.z[l]);
      float* bl = V(y.bv[l]);
      float* dl = V(y.dl[l]);
      block_gemm<true>(
          n, nl, nu, [=](int j, int r) { return du[j * nu + r]; },
          [=](int r, int cc) { return Wu[(int64_t)r * nl + cc]; }, kB_NMAJOR,
          [=](int j, int cc) { return zl[j * nl + cc]; },
          [=](int j, int cc, float x, float zz, bool ok) {
            if (ok) {
              bl[j * nl + cc] = x;
              dl[j * nl + cc] = x * dsilu(zz);
            }
          });
    }

    // ---- the reads, forward (what their backward needs) ----
    if (reads) {
      for (int l = 1; l <= L; ++l) {
        const int nin = p.w[l - 1], nout = p.w[l];
        const float* Wl = W + p.off[l];
        const float* Sl = S + p.off[l];
        const float* h = V(y.h[l - 1]);
        float* hn = V(y.h[l < L ? l : 0]);
        float* zq = V(y.zq[l < L ? l : 1]);
        if (cstart) {
          if (l == L) break;
          block_gemm<true>(
              n, nout, nin, [=](int t, int cc) { return h[t * nin + cc]; },
              [=](int cc, int r) { return Wl[(int64_t)r * nin + cc]; }, kB_KMAJOR,
              [=](int t, int r, float x, bool ok) {
                if (ok) {
                  zq[t * nout + r] = x;
                  hn[t * nout + r] = silu(x);
                }
              });
          continue;
        }
        const float* ak = V(y.act[l - 1]);
        float* sc = V(y.sc[l]);
        float* uw = V(y.uw[l]);
        float* us = V(y.us[l]);
        // one product for the three that share h: columns [a^{l-1} | W | S]
        block_gemm<true>(
            n, n + 2 * nout, nin, [=](int t, int cc) { return h[t * nin + cc]; },
            [=](int cc, int j) {   // every arm's offset kept in range (only one is read)
              const int ja = j < n ? j : 0, jw = j >= n && j < n + nout ? j - n : 0, js = j >= n + nout ? j - n - nout : 0;
              const float* x = j < n          ? ak + (int64_t)ja * nin + cc
                               : j < n + nout ? Wl + (int64_t)jw * nin + cc
                                              : Sl + (int64_t)js * nin + cc;
              return *x;
            },
            kB_KMAJOR,
            [=](int t, int j, float x, bool ok) {
              if (!ok) return;
              if (j < n)
                sc[t * bb + j] = x;
              else if (j < n + nout)
                uw[t * nout + j - n] = x;
              else
                us[t * nout + j - n - nout] = x;
            });
        if (l == L) break;
        // zq = A uw + F us - (D o sc) delta
        const float* dl = V(y.dl[l]);
        block_gemm<true>(
            n, nout, n,
            [=](int t, int i) {
              const float dv = cD[t * bb + i], sv = sc[t * bb + i];
              return i <= t ? dv * sv : 0.f;
            },
            [=](int i, int r) { return dl[i * nout + r]; }, kB_NMAJOR,
            [=](int t, int r) { return cA[t] * uw[t * nout + r] + cF[t] * us[t * nout + r]; },
            [=](int t, int r, float x, float base, bool ok) {
              const float zv = base - x;
              if (ok) {
                zq[t * nout + r] = zv;
                hn[t * nout + r] = silu(zv);
              }
            });
      }

      // ---- the reads, backward (top layer down) ----
      for (int l = L; l >= 1; --l) {
        const int nin = p.w[l - 1], nout = p.w[l];
        const float* Wl = W + p.off[l];
        const float* Sl = S + p.off[l];
        const float* rho = V(y.rho[l]);
        const float* h = V(y.h[l - 1]);
        const bool first = l == 1;
        float* rdn = V(y.rho[first ? l : l - 1]);        // used below layer 1 only
        const float* zqd = V(y.zq[first ? 1 : l - 1]);   // used below layer 1 only
        float* dqc = p.dq + row0 * d;
        // hbar -> rho^{l-1} (or qbar)
        auto hbar_pre = [=](int t, int cc) { return first ? 0.f : zqd[t * nin + cc]; };
        auto hbar_epi = [=](int t, int cc, float x, float zz, bool ok) {
          if (first) {
            if (ok) dqc[t * d + cc] = x;
          } else if (ok) {
            rdn[t * nin + cc] = x * dsilu(zz);
          }
        };
        if (cstart) {
          block_gemm<true>(
              n, nin, nout, [=](int t, int r) { return rho[t * nout + r]; },
              [=](int r, int cc) { return Wl[(int64_t)r * nin + cc]; }, kB_NMAJOR, hbar_pre, hbar_epi);
          continue;
        }
        const float* uw = V(y.uw[l]);
        const float* us = V(y.us[l]);
        const float* sc = V(y.sc[l]);
        const float* dl = V(y.dl[l]);
        row_dots(Abar, rho, nout, uw, nout, n, nout);
        row_dots(Fbar, rho, nout, us, nout, n, nout);
        // R = rho delta^T: Dbar, and the masked products -D o R, -D o sc
        block_gemm<true>(
            n, n, nout, [=](int t, int r) { return rho[t * nout + r]; },
            [=](int r, int i) { return dl[i * nout + r]; }, kB_KMAJOR,
            [=](int t, int i) {
              const int64_t e = (int64_t)t * bb + i;
              return make_float3(cD[e], sc[e], Dbar[e]);
            },
            [=](int t, int i, float x, float3 pv, bool ok) {
              const int64_t e = (int64_t)t * bb + i;
              const float dv = pv.x, sv = pv.y, db = pv.z;
              const bool lo = i <= t;
              if (ok) {
                dr[e] = lo ? -dv * x : 0.f;
                dsc[e] = lo ? -dv * sv : 0.f;
                Dbar[e] = lo ? db - x * sv : db;
              }
            });
        // hbar = [A rho | F rho | -D o R] x [W; S; a^{l-1}]
        const float* ak = V(y.act[l - 1]);
        block_gemm<true>(
            n, nin, 2 * nout + n,
            [=](int t, int kk) {
              const bool st = kk < 2 * nout;   // every arm's offset kept in range (only one is read)
              const int kr = kk < nout ? kk : (st ? kk - nout : 0), kd = st ? 0 : kk - 2 * nout;
              const float* x = st ? rho + t * nout + kr : dr + (int64_t)t * bb + kd;
              const float f = *(kk < nout ? cA + t : cF + t);
              const float v = *x;
              return st ? f * v : v;
            },
            [=](int kk, int cc) {
              const int kw = kk < nout ? kk : 0, ks = kk >= nout && kk < 2 * nout ? kk - nout : 0,
                        ka = kk >= 2 * nout ? kk - 2 * nout : 0;
              const float* x = kk < nout       ? Wl + (int64_t)kw * nin + cc
                               : kk < 2 * nout ? Sl + (int64_t)ks * nin + cc
                                               : ak + (int64_t)ka * nin + cc;
              return *x;
            },
            kB_NMAJOR, hbar_pre, hbar_epi);
        // deltabar^l += (-D o sc)^T rho,  abar^{l-1} += (-D o R)^T h^{l-1}
        float* dbl = V(y.dbar[l]);
        float* abl = V(y.abar[l - 1]);
        block_gemm<false>(
            n, nout, n, [=](int i, int t) { return dsc[(int64_t)t * bb + i]; },
            [=](int t, int r) { return rho[t * nout + r]; }, kB_NMAJOR,
            [=](int i, int r) { return dbl[i * nout + r]; },
            [=](int i, int r, float x, float o, bool ok) {
              if (ok) dbl[i * nout + r] = o + x;
            });
        block_gemm<false>(
            n, nin, n, [=](int i, int t) { return dr[(int64_t)t * bb + i]; },
            [=](int t, int cc) { return h[t * nin + cc]; }, kB_NMAJOR,
            [=](int i, int cc) { return abl[i * nin + cc]; },
            [=](int i, int cc, float x, float o, bool ok) {
              if (ok) abl[i * nin + cc] = o + x;
            });
      }
    }

  }   // kProduce
  if (phase == kConsume) {
    // ---- the fold's adjoint (Wbar, Sbar of the chunk end) ----
    for (int l = 1; l <= L; ++l) {
      const int nin = p.w[l - 1], nout = p.w[l];
      const float* Wbl = Wb + p.off[l];
      const float* Sbl = Sb + p.off[l];
      const float* ak = V(y.act[l - 1]);
      const float* dl = V(y.dl[l]);
      float* dbl = V(y.dbar[l]);
      float* abl = V(y.abar[l - 1]);
      const float* Dn = cD + (int64_t)(n - 1) * bb;
      // Wbar a_i and Sbar a_i in one product: columns [Wbar | Sbar]
      block_gemm<true>(
          n, 2 * nout, nin, [=](int i, int cc) { return ak[i * nin + cc]; },
          [=](int cc, int j) {
            const int jw = j < nout ? j : 0, js = j < nout ? 0 : j - nout;
            return *(j < nout ? Wbl + (int64_t)jw * nin + cc : Sbl + (int64_t)js * nin + cc);
          },
          kB_KMAJOR,
          [=](int i, int j, float x, bool ok) {
            if (!ok) return;
            if (j < nout)
              xw[i * mw + j] = x;
            else
              xs[i * mw + j - nout] = x;
          });
      // deltabar_i -= D[n-1,i] xw_i + U_i xs_i;  Dbar[n-1,i], Ubar_i from delta_i . (xw_i, xs_i)
      each(
          n * nout,
          [&](int e) {
            const int i = e / nout, r = e % nout;
            return dbl[e] - (Dn[i] * xw[i * mw + r] + cU[i] * xs[i * mw + r]);
          },
          [&](int e, float x) { dbl[e] = x; });
      row_dots(Dbar + (int64_t)(n - 1) * bb, dl, nout, xw, mw, n, nout, -1.f);
      row_dots(Ubar, dl, nout, xs, mw, n, nout, -1.f);
      // abar^{l-1} -= [D[n-1,i] delta_i | U_i delta_i] x [Wbar; Sbar]
      block_gemm<true>(
          n, nin, 2 * nout,
          [=](int i, int kk) {
            const float f = *(kk < nout ? Dn + i : cU + i);
            return -f * dl[i * nout + (kk < nout ? kk : kk - nout)];
          },
          [=](int kk, int cc) {
            const int kw = kk < nout ? kk : 0, ks = kk < nout ? 0 : kk - nout;
            return *(kk < nout ? Wbl + (int64_t)kw * nin + cc : Sbl + (int64_t)ks * nin + cc);
          },
          kB_NMAJOR,
          [=](int i, int cc) { return abl[i * nin + cc]; },
          [=](int i, int cc, float x, float o, bool ok) {
            if (ok) abl[i * nin + cc] = o + x;
          });
    }

    // ---- backward of the inner gradient (second-order terms) ----
    for (int l = 1; l < L; ++l) {
      const int nl = p.w[l], nu = p.w[l + 1];
      const float* dbl = V(y.dbar[l]);
      const float* zl = V(y.z[l]);
      const float* bl = V(y.bv[l]);
      float* bbl = V(y.bbar[l]);
      float* zbl = V(y.zbar[l]);
      each(
          n * nl,
          [&](int e) {
            const float db = dbl[e], zz = zl[e];
            return make_float2(db * dsilu(zz), db * bl[e] * d2silu(zz));
          },
          [&](int e, float2 x) {
            bbl[e] = x.x;
            zbl[e] = x.y;
          });
      __syncthreads();
      const float* Wu = W + p.off[l + 1];
      float* dbu = V(y.dbar[l + 1]);
      block_gemm<true>(
          n, nu, nl, [=](int i, int cc) { return bbl[i * nl + cc]; },
          [=](int cc, int r) { return Wu[(int64_t)r * nl + cc]; }, kB_KMAJOR,
          [=](int i, int r) { return dbu[i * nu + r]; },
          [=](int i, int r, float x, float o, bool ok) {
            if (ok) dbu[i * nu + r] = o + x;
          });
    }
    {
      const float* dbL = V(y.dbar[L]);
      each(n * d, [&](int e) { return -dbL[e]; }, [&](int e, float x) { p.dv[row0 * d + e] = x; });
    }
    for (int l = L; l >= 1; --l) {
      const int nin = p.w[l - 1], nout = p.w[l];
      float* zbl = l == L ? V(y.dbar[L]) : V(y.zbar[l]);
      if (l < L) {
        const float* abl = V(y.abar[l]);
        const float* zl = V(y.z[l]);
        each(n * nout, [&](int e) { return zbl[e] + abl[e] * dsilu(zl[e]); }, [&](int e, float x) { zbl[e] = x; });
        __syncthreads();
      }
      const float* Wl = W + p.off[l];
      float* abd = V(y.abar[l - 1]);
      block_gemm<true>(
          n, nin, nout, [=](int i, int r) { return zbl[i * nout + r]; },
          [=](int r, int cc) { return Wl[(int64_t)r * nin + cc]; }, kB_NMAJOR,
          [=](int i, int cc) { return abd[i * nin + cc]; },
          [=](int i, int cc, float x, float o, bool ok) {
            if (ok) abd[i * nin + cc] = o + x;
          });
    }
    {
      const float* ab0 = V(y.abar[0]);
      each(n * d, [&](int e) { return ab0[e]; }, [&](int e, float x) { p.dk[row0 * d + e] = x; });
    }

    // ---- state adjoints: Sbar, then Wbar (both read the chunk-end Wbar) ----
    const float An = cA[n - 1], En = cE[n - 1], Fn = cF[n - 1];
    float sWW = 0.f, sWS = 0.f, sSS = 0.f;   // <Wbar, W>, <Wbar, S>, <Sbar, S>
    for (int l = 1; l <= L; ++l) {
      const int nin = p.w[l - 1], nout = p.w[l];
      float* Wbl = Wb + p.off[l];
      float* Sbl = Sb + p.off[l];
      const float* Wl = W + p.off[l];
      const float* Sl = S + p.off[l];
      const float* rho = V(y.rho[l]);
      const float* h = V(y.h[l - 1]);
      auto sbar_pre = [=](int r, int cc) {
        const int64_t e = (int64_t)r * nin + cc;
        return make_float4(Wbl[e], Sbl[e], Wl[e], Sl[e]);
      };
      auto sbar_epi = [&](int r, int cc, float x, float4 pv, bool ok) {
        const int64_t e = (int64_t)r * nin + cc;
        const float wbv = pv.x, sbv = pv.y, wv = pv.z, sv = pv.w;
        if (ok) {
          Sbl[e] = Fn * wbv + En * sbv + x;
          sWW += wbv * wv;
          sWS += wbv * sv;
          sSS += sbv * sv;
        }
      };
      if (reads && !cstart) {
        block_gemm<false>(
            nout, nin, n, [=](int r, int t) { return cF[t] * rho[t * nout + r]; },
            [=](int t, int cc) { return h[t * nin + cc]; }, kB_NMAJOR, sbar_pre, sbar_epi);
      } else {
        each(
            nout * nin, [&](int e) { return sbar_pre(e / nin, e % nin); },
            [&](int e, float4 pv) { sbar_epi(e / nin, e % nin, 0.f, pv, true); });
        __syncthreads();
      }
      // Wbar <- A_{n-1} Wbar + [rho-part | delta-bbar part | zbar-a part]
      const int kt = reads ? n : 0;
      const int kd = l >= 2 ? n : 0;
      const float* dl = V(y.dl[l]);
      const float* ak = V(y.act[l - 1]);
      const float* bbd = l >= 2 ? V(y.bbar[l - 1]) : ak;   // unused below layer 2
      const float* zbl = l == L ? V(y.dbar[L]) : V(y.zbar[l]);
      const bool unit_t = cstart;
      block_gemm<false>(
          nout, nin, kt + kd + n,
          [=](int r, int kk) {
            const bool pt = kk < kt, pd = !pt && kk < kt + kd;
            const int i = pt ? kk : pd ? kk - kt : kk - kt - kd;
            const float* x = pt ? rho + i * nout + r : pd ? dl + i * nout + r : zbl + i * nout + r;
            const float f = (pt && !unit_t) ? cA[i] : 1.f;
            return f * *x;
          },
          [=](int kk, int cc) {
            const bool pt = kk < kt, pd = !pt && kk < kt + kd;
            const int i = pt ? kk : pd ? kk - kt : kk - kt - kd;
            const float* x = pt ? h + i * nin + cc : pd ? bbd + i * nin + cc : ak + i * nin + cc;
            return *x;
          },
          kB_NMAJOR,
          [=](int r, int cc) { return An * Wbl[(int64_t)r * nin + cc]; },
          [=](int r, int cc, float x, float base, bool ok) {
            if (ok) Wbl[(int64_t)r * nin + cc] = base + x;
          });
    }
    sWW = block_sum(sWW, red);
    sWS = block_sum(sWS, red);
    sSS = block_sum(sSS, red);

    // ---- gate gradients: the coefficient adjoints back through their recurrences ----
    if (tid == 0) {
      Abar[n - 1] += sWW;
      Fbar[n - 1] += sWS;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kBT) {
      // column i of D and P (t > i), and U_i = theta_i P[n-1,i]
      const float ti = th[i * gs];
      float tb = cP[(int64_t)(n - 1) * bb + i] * Ubar[i];
      float dacc = 0.f, pacc = ti * Ubar[i];
      for (int t0 = n - 1; t0 > i; t0 -= kBatch) {
        float db[kBatch], dm[kBatch], pe[kBatch], pm[kBatch], ev[kBatch], av[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = max(t0 - j, i + 1);
          const int64_t e = (int64_t)t * bb + i;
          db[j] = Dbar[e];
          dm[j] = cD[e - bb];
          pe[j] = cP[e];
          pm[j] = cP[e - bb];
          ev[j] = et[t * gs];
          av[j] = al[t * gs];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = t0 - j;
          if (t > i) {
            const int64_t e = (int64_t)t * bb + i;
            dacc += db[j];
            Ca[e] = -dm[j] * dacc;                // D[t,i] = (1 - alpha_t) D[t-1,i] + theta_i P[t,i]
            tb += pe[j] * dacc;
            pacc += ti * dacc;
            Ce[e] = pm[j] * pacc;                 // P[t,i] = eta_t P[t-1,i]
            pacc *= ev[j];
            dacc *= 1.f - av[j];
          }
        }
      }
      dacc += Dbar[(int64_t)i * bb + i];
      gt[i] = tb + dacc;                        // D[i,i] = theta_i
    }
    if (tid == kBT - 1) {   // beside the column recurrences, as in the forward coefficients
      float abar = 0.f, fbar = 0.f, ebar = sSS;
      for (int t0 = n - 1; t0 >= 0; t0 -= kBatch) {
        float am[kBatch], em[kBatch], fm[kBatch], ab[kBatch], fb[kBatch], ev[kBatch], av[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = max(t0 - j, 0), tm = max(t - 1, 0);
          am[j] = t > 0 ? cA[tm] : 1.f;
          em[j] = t > 0 ? cE[tm] : 1.f;
          fm[j] = t > 0 ? cF[tm] : 0.f;
          ab[j] = Abar[t];
          fb[j] = Fbar[t];
          ev[j] = et[t * gs];
          av[j] = al[t * gs];
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int t = t0 - j;
          if (t >= 0) {
            const float a1 = 1.f - av[j];
            abar += ab[j];
            fbar += fb[j];
            ebar += fbar;                         // F_t = (1 - alpha_t) F_{t-1} + E_t
            ga[t] = -am[j] * abar - fm[j] * fbar;  // A_t = (1 - alpha_t) A_{t-1}
            ge[t] = em[j] * ebar;                 // E_t = eta_t E_{t-1}
            abar *= a1;
            fbar *= a1;
            ebar *= ev[j];
          }
        }
      }
    }
    __syncthreads();
    {
      // row sums over i < t of Ca, Ce (rows held in lanes as in row_dots)
      const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      for (int t0 = 0; t0 < n; t0 += kBT) {
        const int jn = min(64, (n - t0 - wv + kBW - 1) / kBW);
        float ha = 0.f, he = 0.f;
        for (int j0 = 0; j0 < jn; j0 += 4) {
          int tu[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) tu[u] = t0 + wv + kBW * min(j0 + u, jn - 1);
          float sa[4] = {0.f, 0.f, 0.f, 0.f}, se[4] = {0.f, 0.f, 0.f, 0.f};
          for (int i = lane; i < tu[3]; i += 64) {   // tu[3] is the group's longest row
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float xa = Ca[(int64_t)tu[u] * bb + i], xe = Ce[(int64_t)tu[u] * bb + i];
              sa[u] += i < tu[u] ? xa : 0.f;
              se[u] += i < tu[u] ? xe : 0.f;
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float ra = wave_sum(sa[u]), re = wave_sum(se[u]);
            ha = lane == j0 + u ? ra : ha;
            he = lane == j0 + u ? re : he;
          }
        }
        const int t = t0 + wv + kBW * lane;
        if (t < n) {
          ga[t] += ha;
          ge[t] += he;
        }
      }
    }
    __syncthreads();
    if (p.chunk_gates) {
      float sa = 0.f, se = 0.f, st = 0.f;
      for (int t = tid; t < n; t += kBT) {
        sa += ga[t];
        se += ge[t];
        st += gt[t];
      }
      sa = block_sum(sa, red);
      se = block_sum(se, red);
      st = block_sum(st, red);
      if (tid == 0) {
        p.dalpha[g0] = sa;
        p.deta[g0] = se;
        p.dtheta[g0] = st;
      }
    } else {
      for (int t = tid; t < n; t += kBT) {
        p.dalpha[g0 + t] = ga[t];
        p.deta[g0 + t] = ge[t];
        p.dtheta[g0 + t] = gt[t];
      }
    }
  }   // kConsume
}

BwLayout bw_layout(const Shape& s, int b) {
  BwLayout y{};
  int64_t cur = 0;
  auto take = [&](int64_t n) {
    const int64_t o = cur;
    cur += (n + 3) / 4 * 4;
    return o;
  };
  const int L = s.L;
  for (int l = 0; l <= L; ++l) y.act[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l < L; ++l) y.z[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l <= L; ++l) y.dl[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l < L; ++l) y.bv[l] = take((int64_t)b * s.widths[l]);
  for (int l = 0; l < L; ++l) y.h[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l < L; ++l) y.zq[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l <= L; ++l) y.uw[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l <= L; ++l) y.us[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l <= L; ++l) y.rho[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l <= L; ++l) y.sc[l] = take((int64_t)b * b);
  for (int l = 1; l <= L; ++l) y.dbar[l] = take((int64_t)b * s.widths[l]);
  for (int l = 0; l < L; ++l) y.abar[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l < L; ++l) y.bbar[l] = take((int64_t)b * s.widths[l]);
  for (int l = 1; l < L; ++l) y.zbar[l] = take((int64_t)b * s.widths[l]);
  y.vin = take((int64_t)b * s.d);
  y.xw = take((int64_t)b * s.maxw);
  y.xs = take((int64_t)b * s.maxw);
  y.dsc = take((int64_t)b * b);
  y.dr = take((int64_t)b * b);
  y.D = take((int64_t)b * b);
  y.P = take((int64_t)b * b);
  y.Dbar = take((int64_t)b * b);
  y.Ca = take((int64_t)b * b);
  y.Ce = take((int64_t)b * b);
  y.A = take(b);
  y.E = take(b);
  y.F = take(b);
  y.U = take(b);
  y.Abar = take(b);
  y.Fbar = take(b);
  y.Ubar = take(b);
  y.ga = take(b);
  y.ge = take(b);
  y.gt = take(b);
  y.red = take(64);
  y.total = cur;
  return y;
}

int rows_per_chunk(const Shape& s, int chunk) { return chunk < s.N ? chunk : s.N; }

int64_t bw_region_floats(const Shape& s, int b) { return (bw_layout(s, b).total + 63) / 64 * 64; }


}  // namespace

namespace {
std::mutex g_side_mu;
SideStream g_side[64];
}  // namespace

hipError_t side_stream(int dev, SideStream** out, std::unique_lock<std::mutex>& lock) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  lock = std::unique_lock<std::mutex>(g_side_mu);
  if (!g_side[dev].st) {
    SideStream x;
    hipError_t e = hipStreamCreateWithFlags(&x.st, hipStreamNonBlocking);
    hipEvent_t* evs[6] = {&x.fork, &x.join, &x.prod[0], &x.prod[1], &x.cons[0], &x.cons[1]};
    for (int i = 0; i < 6 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(evs[i], hipEventDisableTiming);
    if (e != hipSuccess) return e;   // (what was created is kept: a few handles)
    g_side[dev] = x;
  }
  *out = &g_side[dev];
  return hipSuccess;
}

hipError_t join_side(SideStream* x, hipStream_t stream, hipError_t err) {
  hipError_t e = hipEventRecord(x->join, x->st);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, x->join, 0);
  if (e != hipSuccess) (void)hipGetLastError();   // (cleared, so the first error is the one reported)
  return err != hipSuccess ? err : e;
}

bool backward_supported(const Shape& s, int chunk) {
  // the chunk bound of the forward sweep (the generic kernel); it also keeps
  // every [b x b] index inside int
  if (chunk < 1 || chunk > kMaxChunkGeneric || s.N < 1) return false;
  if (s.maxw > kMaxWidthBackward) return false;
  for (int l = 0; l <= s.L; ++l)
    if (s.widths[l] % 4 != 0) return false;
  return true;
}

int64_t backward_ws_floats_per_stream(const Shape& s, int chunk) {
  const int64_t nchunks = (s.N + chunk - 1) / chunk;
  const int b = rows_per_chunk(s, chunk);
  // the forward sweep's workspace and the reverse sweep's two regions share
  // the space after the checkpoints (the sweep ends before the reverse starts)
  const int64_t region = std::max(2 * bw_region_floats(s, b), generic_ws_floats_per_stream(s, b));
  return nchunks * 2 * s.P + (region + 63) / 64 * 64;
}

hipError_t launch_backward(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                           const float* alpha, const float* eta, const float* theta, const float* W_in,
                           const float* S_in, const float* dy, const float* dW_out, const float* dS_out, float* dk,
                           float* dv, float* dq, float* dalpha, float* deta, float* dtheta, float* dW_in,
                           float* dS_in, float* ws, hipStream_t stream) {
  BwdParams p{};
  p.N = s.N;
  p.chunk = chunk;
  p.nchunks = (s.N + chunk - 1) / chunk;
  p.b = rows_per_chunk(s, chunk);
  p.L = s.L;
  p.d = s.d;
  p.io = s.io;
  p.read_mode = s.read_mode;
  p.chunk_gates = s.chunk_gates;
  for (int l = 0; l <= s.L; ++l) p.w[l] = s.widths[l];
  for (int l = 1; l <= s.L; ++l) p.off[l] = s.off[l];
  p.P = s.P;
  p.maxw = s.maxw;
  p.k = k; p.v = v; p.q = q;
  p.alpha = alpha; p.eta = eta; p.theta = theta;
  p.dy = dy; p.dW_out = dW_out; p.dS_out = dS_out;
  p.dk = dk; p.dv = dv; p.dq = dq;
  p.dalpha = dalpha; p.deta = deta; p.dtheta = dtheta;
  p.dW_in = dW_in; p.dS_in = dS_in;
  p.ws = ws;
  p.ws_stream = backward_ws_floats_per_stream(s, chunk);
  p.o_buf = (int64_t)p.nchunks * 2 * s.P;
  p.region = bw_region_floats(s, p.b);
  p.lay = bw_layout(s, p.b);
  // forward sweep: the chunk-start states into the checkpoints; its running
  // state lives in dW_in, dS_in (re-initialised by the reverse sweep)
  hipError_t err = launch_generic_checkpoints(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, dW_in, dS_in, s.P,
                                              ws, p.ws_stream, ws + p.o_buf, p.ws_stream, stream);
  if (err != hipSuccess) return err;
  // reverse sweep: chunk c's first phase on the side stream after the second
  // phase of chunk c + 2 (which used the same region), its second phase on
  // the caller's stream after its first phase; the last first phase is also
  // the side stream's last work, so the caller's stream has joined it at the end
  int dev = 0;
  if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
  std::unique_lock<std::mutex> lock;
  SideStream* x = nullptr;
  if ((err = side_stream(dev, &x, lock)) != hipSuccess) return err;
  if ((err = hipEventRecord(x->fork, stream)) != hipSuccess) return err;
  if ((err = hipStreamWaitEvent(x->st, x->fork, 0)) != hipSuccess) return err;
  auto reverse = [&]() -> hipError_t {
    hipError_t e;
    for (int c = p.nchunks - 1; c >= 0; --c) {
      if (c + 2 < p.nchunks && (e = hipStreamWaitEvent(x->st, x->cons[c & 1], 0)) != hipSuccess) return e;
      hipLaunchKernelGGL(backward_kernel, dim3(s.streams), dim3(kBT), 0, x->st, p, c, (int)kProduce);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(x->prod[c & 1], x->st)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(stream, x->prod[c & 1], 0)) != hipSuccess) return e;
      hipLaunchKernelGGL(backward_kernel, dim3(s.streams), dim3(kBT), 0, stream, p, c, (int)kConsume);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(x->cons[c & 1], stream)) != hipSuccess) return e;
    }
    return hipSuccess;
  };
  return join_side(x, stream, reverse());
}

}  // namespace titans
