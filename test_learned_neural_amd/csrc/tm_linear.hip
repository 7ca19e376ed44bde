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
// The rows of a linear memory are independent: row r of W and S is updated
// from delta_j[r] and the shared k_j, and y_j[r] reads only row r.  So a
// stream runs on d / 4 workgroups, each owning four rows of W and S in LDS
// and computing the shared parts (gates, coefficients, the masked scores)
// itself.  Within a workgroup, thread (t, r, quarter) forms the partial
// products of token t and row r over a quarter of the columns, and the four
// partials of a (t, r) pair are summed across neighbouring lanes.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

#include <algorithm>

namespace titans {
namespace {

constexpr int kLT = 256;       // threads per workgroup
constexpr int kLMaxD = 64;
constexpr int kLMaxB = 64;
constexpr int kLRows = 4;      // rows of W and S per workgroup

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
#pragma unroll 4
  for (int c = 0; c < n; c += 4) {
    const float4 x = *(const float4*)(a + c), y = *(const float4*)(b + c);
    s0 = fmaf(x.x, y.x, s0);
    s1 = fmaf(x.y, y.y, s1);
    s2 = fmaf(x.z, y.z, s2);
    s3 = fmaf(x.w, y.w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

// a . b over the n floats of one column quarter (no alignment assumed)
__device__ __forceinline__ float dot1(const float* a, const float* b, int n) {
  float s0 = 0.f, s1 = 0.f;
  int c = 0;
  for (; c + 1 < n; c += 2) {
    s0 = fmaf(a[c], b[c], s0);
    s1 = fmaf(a[c + 1], b[c + 1], s1);
  }
  if (c < n) s0 = fmaf(a[c], b[c], s0);
  return s0 + s1;
}

// the sum over the four lanes of a quad (lanes 4m .. 4m + 3), in every one of them
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  return x;
}

// Barrier for LDS traffic only: this thread's LDS operations complete, then
// s_barrier.  Threads never exchange data through global memory here, so
// the barrier does not wait for global loads (the next chunk's inputs stay
// in flight across it), as a full __syncthreads() fence would.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ void __launch_bounds__(kLT) linear_kernel(LinParams p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int r0 = kLRows * blockIdx.y;   // this workgroup's first row
  const int d = p.d, b = min(p.chunk, p.N);
  const int R = d + 4;           // row stride of the d-wide arrays (16-byte rows)
  const int RB = b + 1;          // row stride of the [b x b] arrays
  float* W = lds;                // [kLRows][R]: W[r0 + rr][c]
  float* S = W + kLRows * R;
  float* K = S + kLRows * R;     // [b][R]: k_j
  float* Q = K + b * R;
  float* V = Q + b * R;          // [b][kLRows]: v_j[r0 + rr]
  float* Dl = V + b * kLRows;    // [b][kLRows]: delta_j[r0 + rr]
  float* Dm = Dl + b * kLRows;   // [b][RB]: D[j][i]
  float* SC = Dm + b * RB;       // D[j][i] (k_i . q_j), i <= j
  float* cA = SC + b * RB;
  float* cE = cA + b;
  float* cF = cE + b;
  float* cU = cF + b;
  float* gA = cU + b;            // the chunk's gates: 1 - alpha, eta, theta
  float* gE = gA + b;
  float* gT = gE + b;
  const int64_t P = (int64_t)d * d;
  const float* Wi = p.W_in + (int64_t)s * P + (int64_t)r0 * d;
  const float* Si = p.S_in + (int64_t)s * P + (int64_t)r0 * d;
  for (int e = tid; e < kLRows * d; e += kLT) {
    W[(e / d) * R + e % d] = Wi[e];
    S[(e / d) * R + e % d] = Si[e];
  }
  // thread (t, rr, qt): token group t = tid / 16, row r0 + rr, column quarter qt
  const int tq = tid >> 4, rr = (tid >> 2) & 3, qt = tid & 3;
  const int dq = d / 4, c0q = qt * dq;
  const bool dq4 = (dq & 3) == 0;   // the quarters are whole 16-byte pieces
  const bool raw = p.read_mode != TM_READ_CHUNK_START;
  const int64_t tok0 = (int64_t)s * p.N;
  const int nch = (p.N + p.chunk - 1) / p.chunk;
  // A chunk's inputs in registers, one thread's share (element tid + kLT m
  // of the chunk's k and q rows, of its v entries for this workgroup's rows,
  // and the gates of token tid): loaded one chunk ahead, so the loads of
  // chunk c + 1 are in flight while chunk c is computed.
  constexpr int kLPre = kLMaxB * kLMaxD / kLT;
  float pk[kLPre], pq[kLPre], pv = 0.f, pa = 0.f, pe = 1.f, pt = 0.f;
  auto load_chunk = [&](int c0) {
    const int n = min(p.chunk, p.N - c0);
#pragma unroll
    for (int m = 0; m < kLPre; ++m) {
      const int e = tid + kLT * m;
      if (e < n * d) {
        const int64_t gi = (tok0 + c0) * d + e;
        pk[m] = ld_io(p.k, gi, p.io);
        pq[m] = ld_io(p.q, gi, p.io);
      }
    }
    if (tid < n * kLRows) pv = ld_io(p.v, (tok0 + c0 + tid / kLRows) * d + r0 + tid % kLRows, p.io);
    const int64_t g0 = p.chunk_gates ? (int64_t)s * nch + c0 / p.chunk : tok0 + c0;
    const int gs = p.chunk_gates ? 0 : 1;
    if (tid < n) {
      pa = p.alpha[g0 + tid * gs];
      pe = p.eta[g0 + tid * gs];
      pt = p.theta[g0 + tid * gs];
    }
  };
  if (p.N > 0) load_chunk(0);
  for (int c0 = 0; c0 < p.N; c0 += p.chunk) {
    const int n = min(p.chunk, p.N - c0);
    lds_barrier();   // the previous fold is complete
    // ---- the chunk's rows (fp32) and its coefficients ----
#pragma unroll
    for (int m = 0; m < kLPre; ++m) {
      const int e = tid + kLT * m;
      if (e < n * d) {
        K[(e / d) * R + e % d] = pk[m];
        Q[(e / d) * R + e % d] = pq[m];
      }
    }
    if (tid < n * kLRows) V[tid] = pv;
    if (tid < n) {
      gA[tid] = 1.f - pa;
      gE[tid] = pe;
      gT[tid] = pt;
    }
    if (c0 + p.chunk < p.N) load_chunk(c0 + p.chunk);
    lds_barrier();
    if (tid < n) {   // column i of D (rows i..n-1) and U_i
      const int i = tid;
      const float ti = gT[i];
      float di = ti, pr = 1.f;
      for (int t = 0; t < i; ++t) Dm[t * RB + i] = 0.f;
      Dm[i * RB + i] = di;
      // the rows' gates read four steps ahead, so the recurrence does not
      // wait on an LDS read per step
      int t = i + 1;
      for (; t + 4 <= n; t += 4) {
        float av[4], ev[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          av[u] = gA[t + u];
          ev[u] = gE[t + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pr *= ev[u];
          di = av[u] * di + ti * pr;
          Dm[(t + u) * RB + i] = di;
        }
      }
      for (; t < n; ++t) {
        pr *= gE[t];
        di = gA[t] * di + ti * pr;
        Dm[t * RB + i] = di;
      }
      cU[i] = ti * pr;
    } else if (tid >= kLT - 64) {   // A, E, F: prefix scans over the chunk's tokens on the last wave
      const int l = tid - (kLT - 64);
      const float om = l < n ? gA[l] : 1.f, et = l < n ? gE[l] : 1.f;
      // E_l = prod_{m<=l} eta_m; (A_l, F_l) = the composition of the maps
      // u -> (1 - alpha_m) u + E_m for m <= l, applied to 0
      float e = et;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        const float o = __shfl_up(e, sh);
        if (l >= sh) e *= o;
      }
      float a = om, f = e;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        const float ao = __shfl_up(a, sh), fo = __shfl_up(f, sh);
        if (l >= sh) {
          f = fmaf(a, fo, f);
          a *= ao;
        }
      }
      if (l < n) {
        cA[l] = a;
        cE[l] = e;
        cF[l] = f;
      }
    }
    // ---- residuals of this workgroup's rows at W_0 (four partials per (t, r)) ----
    for (int t = tq; t < n; t += kLT / 16) {
      const float part = dq4 ? dot4(K + t * R + c0q, W + rr * R + c0q, dq) : dot1(K + t * R + c0q, W + rr * R + c0q, dq);
      const float dl = quad_sum(part) - V[t * kLRows + rr];
      if (qt == 0) Dl[t * kLRows + rr] = dl;
    }
    lds_barrier();
    // ---- the masked scores (every workgroup of the stream forms all of them) ----
    if (raw)
      for (int e = tid; e < n * n; e += kLT) {
        const int t = e / n, i = e % n;
        SC[t * RB + i] = i <= t ? Dm[t * RB + i] * dot4(K + i * R, Q + t * R, d) : 0.f;
      }
    lds_barrier();
    // ---- the reads of this workgroup's rows: quarter qt contributes its
    // columns' share of A_t W_0 q_t + F_t S_0 q_t and the masked terms of
    // tokens i = qt, qt + 4, ... ----
    for (int t = tq; t < n; t += kLT / 16) {
      const float yw = dq4 ? dot4(Q + t * R + c0q, W + rr * R + c0q, dq) : dot1(Q + t * R + c0q, W + rr * R + c0q, dq);
      float part;
      if (raw) {
        const float ys = dq4 ? dot4(Q + t * R + c0q, S + rr * R + c0q, dq) : dot1(Q + t * R + c0q, S + rr * R + c0q, dq);
        float g = 0.f;
        for (int i = qt; i <= t; i += 4) g = fmaf(SC[t * RB + i], Dl[i * kLRows + rr], g);
        part = cA[t] * yw + cF[t] * ys - g;
      } else {
        part = yw;
      }
      const float yv = quad_sum(part);
      if (qt == 0) {
        const int64_t o = (tok0 + c0 + t) * d + r0 + rr;
        if (p.io == TM_IO_BF16)
          ((__hip_bfloat16*)p.y)[o] = __float2bfloat16(yv);
        else
          ((float*)p.y)[o] = yv;
      }
    }
    lds_barrier();   // every read of W_0, S_0 is done
    // ---- fold: each thread updates its own elements of this workgroup's rows in place ----
    {
      const float An = cA[n - 1], En = cE[n - 1], Fn = cF[n - 1];
      const float* Dn = Dm + (n - 1) * RB;
      for (int e = tid; e < kLRows * d; e += kLT) {
        const int u = e / d, c = e % d;
        float gd = 0.f, gu = 0.f;
#pragma unroll 4
        for (int j = 0; j < n; ++j) {
          const float dl = Dl[j * kLRows + u], kv = K[j * R + c];
          gd = fmaf(Dn[j] * dl, kv, gd);
          gu = fmaf(cU[j] * dl, kv, gu);
        }
        const float w0 = W[u * R + c], s0 = S[u * R + c];
        W[u * R + c] = An * w0 + Fn * s0 - gd;
        S[u * R + c] = En * s0 - gu;
      }
    }
  }
  lds_barrier();
  float* Wo = p.W_out + (int64_t)s * P + (int64_t)r0 * d;
  float* So = p.S_out + (int64_t)s * P + (int64_t)r0 * d;
  for (int e = tid; e < kLRows * d; e += kLT) {
    Wo[e] = W[(e / d) * R + e % d];
    So[e] = S[(e / d) * R + e % d];
  }
}

int linear_lds_bytes(int d, int b) {
  return (int)sizeof(float) * (2 * kLRows * (d + 4) + 2 * b * (d + 4) + 2 * b * kLRows + 2 * b * (b + 1) + 7 * b);
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
  hipLaunchKernelGGL(linear_kernel, dim3(s.streams, s.d / kLRows), dim3(kLT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace titans
