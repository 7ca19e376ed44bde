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
// intermediates in a per-stream workspace; every contraction is an fp32 FMA
// tile loop staged through LDS.  This path serves any shape and the fp32-io
// linear memory, and is the fallback where no specialised kernel exists.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

namespace titans {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

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
  float* ckpt;        // optional: (W, S) at every chunk start, [chunk][W | S] per stream
  int64_t ckpt_stride;    // floats between streams in ckpt
  float* ws;
  int64_t ws_stride;  // floats per stream
};

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

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C[M x N] = sum_k A(m, k) B(k, n), handed to epi(m, n, value).  The whole
// workgroup cooperates; operands come through accessors (global/L2 reads)
// and are staged through LDS in kGk x 64 k-major tiles, the next tile's
// operands loaded into registers while the current one is multiplied.  Each
// of the four waves computes one 32 x 32 quarter of a 64 x 64 output tile
// with the fp32 matrix instruction v_mfma_f32_32x32x2_f32 (lane l supplies
// A[l%32][l/32] and B[l/32][l%32]; accumulator register r holds row
// 8(r/4) + 4(l/32) + r%4, column l%32), so the arithmetic stays fp32.
constexpr int kGk = 32;                                  // k per staged tile
constexpr int kGPer = kTile * kGk / kThreads;             // operand elements per thread per tile
template <class FA, class FB, class FE>
__device__ void block_gemm(int M, int N, int K, FA fa, FB fb, FE epi) {
  __shared__ float As[kGk][kTile + 1];
  __shared__ float Bs[kGk][kTile + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = (wv >> 1) * 32, wn = (wv & 1) * 32;   // this wave's quarter
  const int li = lane & 31, lk = lane >> 5;
  for (int m0 = 0; m0 < M; m0 += kTile) {
    for (int n0 = 0; n0 < N; n0 += kTile) {
      float ra[kGPer], rb[kGPer];
      auto fetch = [&](int k0) {
#pragma unroll
        for (int q = 0; q < kGPer; ++q) {
          const int e = tid + q * kThreads;
          const int mm = e / kGk, ka = e % kGk;        // A element (m0 + mm, k0 + ka)
          ra[q] = (m0 + mm < M && k0 + ka < K) ? fa(m0 + mm, k0 + ka) : 0.f;
          const int kb = e / kTile, nn = e % kTile;    // B element (k0 + kb, n0 + nn)
          rb[q] = (n0 + nn < N && k0 + kb < K) ? fb(k0 + kb, n0 + nn) : 0.f;
        }
      };
      fetch(0);
      f32x16 acc = {};
      for (int k0 = 0; k0 < K; k0 += kGk) {
#pragma unroll
        for (int q = 0; q < kGPer; ++q) {
          const int e = tid + q * kThreads;
          As[e % kGk][e / kGk] = ra[q];
          Bs[e / kTile][e % kTile] = rb[q];
        }
        __syncthreads();
        if (k0 + kGk < K) fetch(k0 + kGk);   // in flight during the products below
#pragma unroll
        for (int kk = 0; kk < kGk; kk += 2)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kk + lk][wm + li], Bs[kk + lk][wn + li], acc, 0, 0, 0);
        __syncthreads();
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 8 * (r >> 2) + 4 * lk + (r & 3), n = n0 + wn + li;
        if (m < M && n < N) epi(m, n, acc[r]);
      }
    }
  }
  __syncthreads();
}

struct Work {
  float* act[kMaxLayers + 1];    // a^0 = K, a^l [b x n_l]
  float* sp[kMaxLayers + 1];     // SiLU'(z^l), l = 1..L-1
  float* delta[kMaxLayers + 1];  // delta^l, l = 1..L
  float* vin;                    // V [b x d]
  float* hq[2];                  // query-side activations, ping-pong [b x maxw]
  float* sc;                     // masked scores [b x b]
  float* D;                      // [b x b]
  float* A;
  float* E;
  float* F;
  float* U;
};

__device__ Work carve(const GParams& p, float* base) {
  Work w;
  float* cur = base;
  const int b = p.b;
  for (int l = 0; l <= p.L; ++l) { w.act[l] = cur; cur += (int64_t)b * p.widths[l]; }
  for (int l = 1; l < p.L; ++l) { w.sp[l] = cur; cur += (int64_t)b * p.widths[l]; }
  for (int l = 1; l <= p.L; ++l) { w.delta[l] = cur; cur += (int64_t)b * p.widths[l]; }
  w.vin = cur; cur += (int64_t)b * p.d;
  w.hq[0] = cur; cur += (int64_t)b * p.maxw;
  w.hq[1] = cur; cur += (int64_t)b * p.maxw;
  w.sc = cur; cur += (int64_t)b * b;
  w.D = cur; cur += (int64_t)b * b;
  w.A = cur; cur += b;
  w.E = cur; cur += b;
  w.F = cur; cur += b;
  w.U = cur; cur += b;
  return w;
}

__global__ void __launch_bounds__(kThreads) generic_kernel(GParams p) {
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = p.d, L = p.L;
  float* W = p.W + (int64_t)s * p.state_stride;
  float* S = p.S + (int64_t)s * p.state_stride;
  const float* Win = p.W_in + (int64_t)s * p.P;
  const float* Sin = p.S_in + (int64_t)s * p.P;
  if (W != Win)
    for (int64_t i = tid; i < p.P; i += kThreads) W[i] = Win[i];
  if (S != Sin)
    for (int64_t i = tid; i < p.P; i += kThreads) S[i] = Sin[i];
  __syncthreads();
  if (p.N == 0) return;
  Work w = carve(p, p.ws + (int64_t)s * p.ws_stride);
  const int64_t tok0 = (int64_t)s * p.N;

  for (int c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int n = min(p.chunk, p.N - c0);
    if (p.ckpt) {
      // the state at this chunk's start (read only here; it is next written
      // by this chunk's fold, many barriers later)
      float* ck = p.ckpt + (int64_t)s * p.ckpt_stride + (int64_t)(c0 / p.chunk) * 2 * p.P;
      for (int64_t i = tid; i < p.P; i += kThreads) {
        ck[i] = W[i];
        ck[p.P + i] = S[i];
      }
    }
    // the chunk's gates: token j at index j * gs (one shared value when the
    // gates are given per chunk)
    const int64_t g0 = p.chunk_gates ? (int64_t)s * ((p.N + p.chunk - 1) / p.chunk) + c0 / p.chunk : tok0 + c0;
    const int gs = p.chunk_gates ? 0 : 1;
    const float* al = p.alpha + g0;
    const float* et = p.eta + g0;
    const float* th = p.theta + g0;

    // ---- load the chunk's keys, values and queries (fp32 copies) ----
    for (int e = tid; e < n * d; e += kThreads) {
      const int64_t gi = (tok0 + c0) * d + e;
      w.act[0][e] = load_io(p.k, gi, p.io);
      w.vin[e] = load_io(p.v, gi, p.io);
      w.hq[0][(e / d) * p.maxw + (e % d)] = load_io(p.q, gi, p.io);
    }
    // ---- a1: coefficient recurrences (one thread per column i of D) ----
    for (int i = tid; i < n; i += kThreads) {
      float di = th[i * gs], pr = 1.f;
      for (int j = 0; j < i; ++j) w.D[j * n + i] = 0.f;
      w.D[i * n + i] = di;
      for (int j = i + 1; j < n; ++j) {
        pr *= et[j * gs];
        di = (1.f - al[j * gs]) * di + th[i * gs] * pr;
        w.D[j * n + i] = di;
      }
      w.U[i] = th[i * gs] * pr;
    }
    if (tid == 0) {
      float a = 1.f, e = 1.f, f = 0.f;
      for (int j = 0; j < n; ++j) {
        a *= 1.f - al[j * gs];
        e *= et[j * gs];
        f = (1.f - al[j * gs]) * f + e;
        w.A[j] = a;
        w.E[j] = e;
        w.F[j] = f;
      }
    }
    __syncthreads();

    // ---- a2: key-side forward at the chunk-start weights ----
    for (int l = 1; l <= L; ++l) {
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = W + p.off[l];
      const float* ain = w.act[l - 1];
      float* aout = w.act[l];
      float* spl = w.sp[l];
      float* dl = w.delta[l];
      const float* vin = w.vin;
      const bool last = (l == L);
      block_gemm(
          n, nout, nin, [=](int j, int c) { return ain[j * nin + c]; },
          [=](int c, int r) { return Wl[(int64_t)r * nin + c]; },
          [=](int j, int r, float z) {
            if (last) {
              aout[j * nout + r] = z;
              dl[j * nout + r] = z - vin[j * nout + r];  // a3: residual M(k) - v
            } else {
              aout[j * nout + r] = silu(z);
              spl[j * nout + r] = silu_prime(z);
            }
          });
    }
    // ---- a3: backprop to every layer's delta ----
    for (int l = L; l >= 2; --l) {
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = W + p.off[l];
      const float* dl = w.delta[l];
      float* dprev = w.delta[l - 1];
      const float* spp = w.sp[l - 1];
      block_gemm(
          n, nin, nout, [=](int j, int r) { return dl[j * nout + r]; },
          [=](int r, int c) { return Wl[(int64_t)r * nin + c]; },
          [=](int j, int c, float x) { dprev[j * nin + c] = x * spp[j * nin + c]; });
    }
    // ---- a5: retrieval ----
    int cur = 0;
    for (int l = 1; l <= L && p.y; ++l) {
      const int nin = p.widths[l - 1], nout = p.widths[l];
      const float* Wl = W + p.off[l];
      const float* Sl = S + p.off[l];
      const float* h = w.hq[cur];
      float* hn = w.hq[cur ^ 1];
      const float* ak = w.act[l - 1];
      const float* dl = w.delta[l];
      const bool last = (l == L);
      const int maxw = p.maxw;
      auto epi = [=](int j, int r, float zq) {
        if (last)
          store_io(p.y, (tok0 + c0 + j) * d + r, zq, p.io);
        else
          hn[j * maxw + r] = silu(zq);
      };
      if (p.read_mode == TM_READ_CHUNK_START) {
        block_gemm(
            n, nout, nin, [=](int j, int c) { return h[j * maxw + c]; },
            [=](int c, int r) { return Wl[(int64_t)r * nin + c]; }, epi);
      } else {
        float* sc = w.sc;
        const float* D = w.D;
        // masked, decay-weighted scores (D o (h a^T)), lower triangle
        block_gemm(
            n, n, nin, [=](int j, int c) { return h[j * maxw + c]; },
            [=](int c, int i) { return ak[i * nin + c]; },
            [=](int j, int i, float x) { sc[j * n + i] = (i <= j) ? D[j * n + i] * x : 0.f; });
        const float* A = w.A;
        const float* F = w.F;
        // zq = diag(A) h W^T + diag(F) h S^T - sc delta, as one contraction
        // over the concatenated index [W-part | S-part | token part]
        block_gemm(
            n, nout, 2 * nin + n,
            [=](int j, int kk) {
              if (kk < nin) return A[j] * h[j * maxw + kk];
              if (kk < 2 * nin) return F[j] * h[j * maxw + kk - nin];
              return -sc[j * n + kk - 2 * nin];
            },
            [=](int kk, int r) {
              if (kk < nin) return Wl[(int64_t)r * nin + kk];
              if (kk < 2 * nin) return Sl[(int64_t)r * nin + kk - nin];
              return dl[(kk - 2 * nin) * nout + r];
            },
            epi);
      }
      cur ^= 1;
    }
    // ---- a4: fold the chunk into the state (after every read of W_0, S_0) ----
    {
      const float An = w.A[n - 1], En = w.E[n - 1], Fn = w.F[n - 1];
      const float* Dlast = w.D + (n - 1) * n;
      const float* U = w.U;
      for (int l = 1; l <= L; ++l) {
        const int nin = p.widths[l - 1], nout = p.widths[l];
        float* Wl = W + p.off[l];
        float* Sl = S + p.off[l];
        const float* dl = w.delta[l];
        const float* ak = w.act[l - 1];
        block_gemm(
            nout, nin, n, [=](int r, int j) { return Dlast[j] * dl[j * nout + r]; },
            [=](int j, int c) { return ak[j * nin + c]; },
            [=](int r, int c, float g) {
              const int64_t i = (int64_t)r * nin + c;
              Wl[i] = An * Wl[i] + Fn * Sl[i] - g;
            });
        block_gemm(
            nout, nin, n, [=](int r, int j) { return U[j] * dl[j * nout + r]; },
            [=](int j, int c) { return ak[j * nin + c]; },
            [=](int r, int c, float g) {
              const int64_t i = (int64_t)r * nin + c;
              Sl[i] = En * Sl[i] - g;
            });
      }
    }
    __syncthreads();
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

int64_t generic_ws_floats_per_stream(const Shape& s, int b) {
  int64_t f = 0;
  for (int l = 0; l <= s.L; ++l) f += (int64_t)b * s.widths[l];       // act
  for (int l = 1; l < s.L; ++l) f += (int64_t)b * s.widths[l];        // sp
  for (int l = 1; l <= s.L; ++l) f += (int64_t)b * s.widths[l];       // delta
  f += (int64_t)b * s.d;                                              // vin
  f += 2 * (int64_t)b * s.maxw;                                       // hq
  f += 2 * (int64_t)b * b;                                            // sc, D
  f += 4 * (int64_t)b;                                                // A, E, F, U
  return (f + 63) / 64 * 64;                                          // keep 256-byte alignment
}

hipError_t launch_generic(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                          const float* alpha, const float* eta, const float* theta,
                          const float* W_in, const float* S_in, void* y, float* W_out,
                          float* S_out, float* ws, hipStream_t stream) {
  GParams p = make_params(s, chunk);
  p.b = chunk < s.N ? chunk : (s.N > 0 ? s.N : 1);
  p.k = k;
  p.v = v;
  p.q = q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.W_in = W_in;
  p.S_in = S_in;
  p.y = y;
  p.W = W_out;
  p.S = S_out;
  p.state_stride = s.P;
  p.ckpt = nullptr;
  p.ckpt_stride = 0;
  p.ws = ws;
  p.ws_stride = generic_ws_floats_per_stream(s, p.b);
  hipLaunchKernelGGL(generic_kernel, dim3(s.streams), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_generic_checkpoints(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                                      const float* alpha, const float* eta, const float* theta, const float* W_in,
                                      const float* S_in, float* W, float* S, int64_t state_stride, float* ckpt,
                                      int64_t ckpt_stride, float* ws, int64_t ws_stride, hipStream_t stream) {
  GParams p = make_params(s, chunk);
  p.b = chunk < s.N ? chunk : (s.N > 0 ? s.N : 1);
  p.k = k;
  p.v = v;
  p.q = q;
  p.alpha = alpha;
  p.eta = eta;
  p.theta = theta;
  p.W_in = W_in;
  p.S_in = S_in;
  p.y = nullptr;
  p.W = W;
  p.S = S;
  p.state_stride = state_stride;
  p.ckpt = ckpt;
  p.ckpt_stride = ckpt_stride;
  p.ws = ws;
  p.ws_stride = ws_stride;
  hipLaunchKernelGGL(generic_kernel, dim3(s.streams), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
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
