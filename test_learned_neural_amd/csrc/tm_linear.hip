// Linear memory (one d x d matrix W, its momentum S) on one workgroup per
// stream, for d <= 64 and chunks of at most 64 tokens: the chunked closed
// form of "Titans: Learning to Memorize at Test Time" (mer.dev notes,
// section 3.2, every gradient of a chunk taken at its start state W_0), with
// the memory M(x) = W x (section 3.1, "Memory Architecture", one layer):
//
//   coefficients  A_j = prod_{m<=j} (1 - alpha_m), E_j = prod_{m<=j} eta_m,
//                 F_j = (1 - alpha_j) F_{j-1} + E_j, U_i = theta_i prod_{m>i} eta_m,
//                 D[j,i] = (1 - alpha_j) D[j-1,i] + theta_i prod_{i<m<=j} eta_m, D[i,i] = theta_i
//   residual      delta_j = W_0 k_j - v_j      (the inner gradient is delta_j k_j^T)
//   reads         y_j = A_j W_0 q_j + F_j S_0 q_j - sum_{i<=j} D[j,i] (k_i . q_j) delta_i
//                 (y_j = W_0 q_j with the chunk-start read)
//   fold          W <- A_n W_0 + F_n S_0 - sum_j D[n-1,j] delta_j k_j^T,
//                 S <- E_n S_0 - sum_j U_j delta_j k_j^T
//
// A chunk of this memory is a few thousand multiply-adds per thread, so the
// workgroup keeps the state and the chunk in LDS and runs every product as
// plain fp32 FMAs (one output element per thread at a time, rows read as
// 16-byte vectors), with five barriers per chunk.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

#include <algorithm>

namespace titans {
namespace {

constexpr int kLT = 256;       // threads per workgroup
constexpr int kLMaxD = 64;
constexpr int kLMaxB = 64;

struct LinParams {
  int N, d, chunk, io, read_mode, chunk_gates;
  const void* k;
  const void* v;
  const void* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  const float* W_in;
  const float* S_in;
  void* y;
  float* W_out;
  float* S_out;
};

__device__ __forceinline__ float ld_io(const void* p, int64_t i, int io) {
  if (io == TM_IO_BF16) return __bfloat162float(((const __hip_bfloat16*)p)[i]);
  return ((const float*)p)[i];
}

// a . b over n floats (n a multiple of 4, both 16-byte aligned, in LDS)
__device__ __forceinline__ float dot4(const float* a, const float* b, int n) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int c = 0; c < n; c += 4) {
    const float4 x = *(const float4*)(a + c), y = *(const float4*)(b + c);
    s0 = fmaf(x.x, y.x, s0);
    s1 = fmaf(x.y, y.y, s1);
    s2 = fmaf(x.z, y.z, s2);
    s3 = fmaf(x.w, y.w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

__global__ void __launch_bounds__(kLT) linear_kernel(LinParams p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int d = p.d, b = min(p.chunk, p.N);
  const int R = d + 4;           // row stride of the d-wide arrays (16-byte rows)
  const int RB = b + 1;          // row stride of the [b x b] arrays
  float* W = lds;                // [d][R]: W[r][c]
  float* S = W + d * R;
  float* K = S + d * R;          // [b][R]: k_j
  float* V = K + b * R;
  float* Q = V + b * R;
  float* Dl = Q + b * R;         // delta_j
  float* Dm = Dl + b * R;        // [b][RB]: D[j][i]
  float* SC = Dm + b * RB;       // D[j][i] (k_i . q_j), i <= j
  float* cA = SC + b * RB;
  float* cE = cA + b;
  float* cF = cE + b;
  float* cU = cF + b;
  float* gA = cU + b;            // the chunk's gates: 1 - alpha, eta, theta
  float* gE = gA + b;
  float* gT = gE + b;
  const int64_t P = (int64_t)d * d;
  const float* Wi = p.W_in + (int64_t)s * P;
  const float* Si = p.S_in + (int64_t)s * P;
  for (int e = tid; e < d * d; e += kLT) {
    W[(e / d) * R + e % d] = Wi[e];
    S[(e / d) * R + e % d] = Si[e];
  }
  const int64_t tok0 = (int64_t)s * p.N;
  const int nch = (p.N + p.chunk - 1) / p.chunk;
  for (int c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int n = min(p.chunk, p.N - c0);
    __syncthreads();   // the previous fold is complete
    // ---- the chunk's rows (fp32) and its coefficients ----
    for (int e = tid; e < n * d; e += kLT) {
      const int64_t gi = (tok0 + c0) * d + e;
      const int j = e / d, c = e % d;
      K[j * R + c] = ld_io(p.k, gi, p.io);
      V[j * R + c] = ld_io(p.v, gi, p.io);
      Q[j * R + c] = ld_io(p.q, gi, p.io);
    }
    const int64_t g0 = p.chunk_gates ? (int64_t)s * nch + c0 / p.chunk : tok0 + c0;
    const int gs = p.chunk_gates ? 0 : 1;
    if (tid < n) {
      gA[tid] = 1.f - p.alpha[g0 + tid * gs];
      gE[tid] = p.eta[g0 + tid * gs];
      gT[tid] = p.theta[g0 + tid * gs];
    }
    __syncthreads();
    if (tid < n) {   // column i of D (rows i..n-1) and U_i
      const int i = tid;
      const float ti = gT[i];
      float di = ti, pr = 1.f;
      for (int t = 0; t < i; ++t) Dm[t * RB + i] = 0.f;
      Dm[i * RB + i] = di;
      for (int t = i + 1; t < n; ++t) {
        pr *= gE[t];
        di = gA[t] * di + ti * pr;
        Dm[t * RB + i] = di;
      }
      cU[i] = ti * pr;
    } else if (tid == kLT - 1) {   // A, E, F
      float a = 1.f, e = 1.f, f = 0.f;
      for (int t = 0; t < n; ++t) {
        const float om = gA[t];
        a *= om;
        e *= gE[t];
        f = om * f + e;
        cA[t] = a;
        cE[t] = e;
        cF[t] = f;
      }
    }
    __syncthreads();
    // ---- residuals at W_0, and the masked scores ----
    for (int e = tid; e < n * d; e += kLT) {
      const int j = e / d, r = e % d;
      Dl[j * R + r] = dot4(K + j * R, W + r * R, d) - V[j * R + r];
    }
    if (p.read_mode != TM_READ_CHUNK_START)
      for (int e = tid; e < n * n; e += kLT) {
        const int t = e / n, i = e % n;
        SC[t * RB + i] = i <= t ? Dm[t * RB + i] * dot4(K + i * R, Q + t * R, d) : 0.f;
      }
    __syncthreads();
    // ---- the reads (chunk-start state and this chunk's gradients), four
    // consecutive outputs of a token per thread ----
    const int d4 = d / 4;
    for (int e = tid; e < n * d4; e += kLT) {
      const int t = e / d4, r = (e % d4) * 4;
      float yw[4] = {0.f, 0.f, 0.f, 0.f}, ys[4] = {0.f, 0.f, 0.f, 0.f};
      const bool raw = p.read_mode != TM_READ_CHUNK_START;
      for (int c = 0; c < d; c += 4) {
        const float4 qv = *(const float4*)(Q + t * R + c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 wv = *(const float4*)(W + (r + u) * R + c);
          yw[u] = fmaf(qv.x, wv.x, fmaf(qv.y, wv.y, fmaf(qv.z, wv.z, fmaf(qv.w, wv.w, yw[u]))));
          if (raw) {
            const float4 sv = *(const float4*)(S + (r + u) * R + c);
            ys[u] = fmaf(qv.x, sv.x, fmaf(qv.y, sv.y, fmaf(qv.z, sv.z, fmaf(qv.w, sv.w, ys[u]))));
          }
        }
      }
      float yv[4] = {yw[0], yw[1], yw[2], yw[3]};
      if (raw) {
        float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i = 0; i <= t; ++i) {
          const float sc = SC[t * RB + i];
          const float4 dv = *(const float4*)(Dl + i * R + r);
          g.x = fmaf(sc, dv.x, g.x);
          g.y = fmaf(sc, dv.y, g.y);
          g.z = fmaf(sc, dv.z, g.z);
          g.w = fmaf(sc, dv.w, g.w);
        }
        const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) yv[u] = cA[t] * yw[u] + cF[t] * ys[u] - gv[u];
      }
      const int64_t o = (tok0 + c0 + t) * d + r;
      if (p.io == TM_IO_BF16) {
        __hip_bfloat16* yo = (__hip_bfloat16*)p.y + o;
#pragma unroll
        for (int u = 0; u < 4; ++u) yo[u] = __float2bfloat16(yv[u]);
      } else {
        *(float4*)((float*)p.y + o) = make_float4(yv[0], yv[1], yv[2], yv[3]);
      }
    }
    __syncthreads();   // every read of W_0, S_0 is done
    // ---- fold: each thread updates its own four elements of a row in place ----
    {
      const float An = cA[n - 1], En = cE[n - 1], Fn = cF[n - 1];
      const float* Dn = Dm + (n - 1) * RB;
      for (int e = tid; e < d * d4; e += kLT) {
        const int r = e / d4, c = (e % d4) * 4;
        float4 gd = make_float4(0.f, 0.f, 0.f, 0.f), gu = gd;
        for (int j = 0; j < n; ++j) {
          const float dl = Dl[j * R + r];
          const float a = Dn[j] * dl, u = cU[j] * dl;
          const float4 kv = *(const float4*)(K + j * R + c);
          gd.x = fmaf(a, kv.x, gd.x); gd.y = fmaf(a, kv.y, gd.y); gd.z = fmaf(a, kv.z, gd.z); gd.w = fmaf(a, kv.w, gd.w);
          gu.x = fmaf(u, kv.x, gu.x); gu.y = fmaf(u, kv.y, gu.y); gu.z = fmaf(u, kv.z, gu.z); gu.w = fmaf(u, kv.w, gu.w);
        }
        float4* wp = (float4*)(W + r * R + c);
        float4* sp = (float4*)(S + r * R + c);
        const float4 w0 = *wp, s0 = *sp;
        *wp = make_float4(An * w0.x + Fn * s0.x - gd.x, An * w0.y + Fn * s0.y - gd.y, An * w0.z + Fn * s0.z - gd.z,
                          An * w0.w + Fn * s0.w - gd.w);
        *sp = make_float4(En * s0.x - gu.x, En * s0.y - gu.y, En * s0.z - gu.z, En * s0.w - gu.w);
      }
    }
  }
  __syncthreads();
  float* Wo = p.W_out + (int64_t)s * P;
  float* So = p.S_out + (int64_t)s * P;
  for (int e = tid; e < d * d; e += kLT) {
    Wo[e] = W[(e / d) * R + e % d];
    So[e] = S[(e / d) * R + e % d];
  }
}

int linear_lds_bytes(int d, int b) {
  return (int)sizeof(float) * (2 * d * (d + 4) + 4 * b * (d + 4) + 2 * b * (b + 1) + 7 * b);
}

}  // namespace

bool linear_supported(const Shape& s, int chunk) {
  return s.L == 1 && s.d >= 4 && s.d <= kLMaxD && s.d % 4 == 0 && chunk >= 1 && chunk <= kLMaxB;
}

hipError_t launch_linear(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                         const float* alpha, const float* eta, const float* theta, const float* W_in,
                         const float* S_in, void* y, float* W_out, float* S_out, hipStream_t stream) {
  LinParams p;
  p.N = s.N;
  p.d = s.d;
  p.chunk = chunk;
  p.io = s.io;
  p.read_mode = s.read_mode;
  p.chunk_gates = s.chunk_gates;
  p.k = k; p.v = v; p.q = q;
  p.alpha = alpha; p.eta = eta; p.theta = theta;
  p.W_in = W_in; p.S_in = S_in;
  p.y = y; p.W_out = W_out; p.S_out = S_out;
  if (s.streams <= 0) return hipSuccess;
  const int lds = linear_lds_bytes(s.d, std::max(1, std::min(chunk, s.N)));
  hipError_t e = hipFuncSetAttribute((const void*)linear_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(linear_kernel, dim3(s.streams), dim3(kLT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace titans
