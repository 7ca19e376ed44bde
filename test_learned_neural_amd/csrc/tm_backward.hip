// Backward pass through the memory: gradients of a loss with respect to
// every input of titans_mem_forward (k, v, q, the gates, W_in, S_in), for
// the outer loop that trains whatever produces those inputs ("Titans:
// Learning to Memorize at Test Time", mer.dev notes, section 3.1
// "Objective": the memory's parameters are the inner loop, the rest of the
// architecture the outer one).
//
// Forward being differentiated, per token t of chunk c (gradients at the
// chunk-start weights W_c, section 3.2; momentum and forgetting of section
// 3.1):
//   g_t = grad of 0.5 ||M_{W_c}(k_t) - v_t||^2 = {delta_l a_{l-1}^T}
//   S_t = eta_t S_{t-1} - theta_t g_t,   W_t = (1 - alpha_t) W_{t-1} + S_t
//   y_t = M_{W_t}(q_t)   (or M_{W_c}(q_t) with the chunk-start read)
// Reverse mode, token by token from the last (adjoints carry a bar):
//   Wbar += retrieval backprop of ybar_t;  qbar_t from the same backprop
//   alphabar_t = -<Wbar, W_{t-1}>;  Sbar += Wbar;  Wbar *= (1 - alpha_t)
//   etabar_t = <Sbar, S_{t-1}>;  thetabar_t = -<Sbar, g_t>
//   W_c receives the derivative of phi = <Gbar, g_t(W_c, k_t, v_t)> with
//   Gbar = -theta_t Sbar (a Hessian-vector product of the inner loss, which
//   also gives kbar_t and vbar_t); Sbar *= eta_t
// and at the start of each chunk Wbar += (what W_c received).  phi's
// derivative is the backward pass of the inner backward pass:
//   u_l = Gbar_l a_{l-1},  r_l = Gbar_l^T delta_l
//   deltabar_1 = u_1;  e_{l-1} = deltabar_{l-1} * s'(z_{l-1});
//   deltabar_l = u_l + W_l e_{l-1};  W_l gets delta_l e_{l-1}^T;
//   zbar_{l-1} gets deltabar_{l-1} * b_{l-1} * s''(z_{l-1})  (b_{l-1} = W_l^T delta_l)
//   vbar = -deltabar_L;  zbar_L = deltabar_L;  then the forward's adjoints
//   top-down with abar_{l-1} = W_l^T zbar_l + r_l, W_l gets zbar_l a_{l-1}^T,
//   zbar_{l-1} gets abar_{l-1} * s'(z_{l-1});  kbar = abar_0.
//
// Execution: one workgroup per stream, fp32 throughout.  A forward sweep
// (the generic kernel's chunked closed form, without retrieval) stores
// (W, S) at every chunk start in the workspace; the reverse sweep
// recomputes each chunk's per-token states W_t, S_t and the key-side
// vectors (z, delta, b at W_c) into the workspace, then walks its tokens
// backwards.  Matrices stay in global memory (L2-resident for the small
// memories); vectors live in LDS.  Matrix-vector products use 16-lane
// groups per row (float4 loads, DPP sums) or column groups with an LDS
// reduction; the state adjoints are updated in one float4 pass per layer
// that folds in every rank-1 term of the step.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

namespace titans {
namespace {

constexpr int kBT = 512;      // threads per workgroup
constexpr int kBW = kBT / 64;

struct BwdParams {
  int N, chunk, nchunks, streams, L, d, io, read_mode, chunk_gates;
  int w[kMaxLayers + 1];
  int64_t off[kMaxLayers + 1];
  int64_t P;
  int maxw, sumn;
  int zo[kMaxLayers + 1];      // offset of layer l's vector (l = 1..L) in a sum-of-widths vector
  const void* k;
  const void* v;
  const void* q;
  const float* alpha;
  const float* eta;
  const float* theta;
  const float* W_in;
  const float* S_in;
  const float* dy;
  const float* dW_out;
  const float* dS_out;
  float* dk;
  float* dv;
  float* dq;
  float* dalpha;
  float* deta;
  float* dtheta;
  float* dW_in;
  float* dS_in;
  float* ws;
  int64_t ws_stream;           // floats per stream
  int64_t o_cw, o_cs, o_tv, o_wb, o_sb, o_wcb;   // offsets (floats) in a stream's region; checkpoints at 0
  int lds_floats;
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
// sum over the aligned 16-lane group (result in every lane of the group)
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = sum16(x);
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
__device__ __forceinline__ float act(float z) { return z * sgm(z); }                       // SiLU
__device__ __forceinline__ float dact(float z) { const float s = sgm(z); return s * (1.f + z * (1.f - s)); }
__device__ __forceinline__ float d2act(float z) {
  const float s = sgm(z);
  return s * (1.f - s) * (2.f + z * (1.f - 2.f * s));
}

// out[i] = sum_j M[i][j] x[j] (M row-major n_out x n_in, n_in % 4 == 0);
// 16 lanes per row, float4 loads.  Ends with a barrier.
__device__ void mv_rows(float* out, const float* M, const float* x, int n_out, int n_in) {
  const int sl = threadIdx.x & 15, gr = threadIdx.x >> 4;
  constexpr int kRowsPerPass = kBT / 16;
  // four row passes at a time, so that four independent loads are in flight
  for (int i0 = 0; i0 < n_out; i0 += 4 * kRowsPerPass) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 4 * sl; j < n_in; j += 64) {
      float4 m[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kRowsPerPass + gr;
        m[u] = i < n_out ? *(const float4*)(M + (int64_t)i * n_in + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const float x0 = x[j], x1 = x[j + 1], x2 = x[j + 2], x3 = x[j + 3];
#pragma unroll
      for (int u = 0; u < 4; ++u) s[u] += m[u].x * x0 + m[u].y * x1 + m[u].z * x2 + m[u].w * x3;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float t = sum16(s[u]);
      const int i = i0 + u * kRowsPerPass + gr;
      if (i < n_out && sl == 0) out[i] = t;
    }
  }
  __syncthreads();
}

// out[j] = sum_i M[i][j] z[i] (+ add[j] if add): column groups of 4, rows
// split over the remaining threads, partial sums reduced through `red`
// (kBT * 4 floats).  Ends with a barrier.
__device__ void mv_cols(float* out, const float* M, const float* z, int n_out, int n_in, float* red,
                        const float* add = nullptr, float add_scale = 0.f) {
  const int cg = n_in / 4;
  if (cg >= kBT) {
    for (int c = threadIdx.x; c < cg; c += kBT) {
      float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = 0; i < n_out; ++i) {
        const float4 m = *(const float4*)(M + (int64_t)i * n_in + 4 * c);
        const float zi = z[i];
        s.x += m.x * zi; s.y += m.y * zi; s.z += m.z * zi; s.w += m.w * zi;
      }
      const float o[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * c + e] = o[e] + (add ? add_scale * add[4 * c + e] : 0.f);
    }
    __syncthreads();
    return;
  }
  const int rg = kBT / cg;                 // row groups
  const int c = threadIdx.x % cg, g = threadIdx.x / cg;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g < rg) {
#pragma unroll 4
    for (int i = g; i < n_out; i += rg) {
      const float4 m = *(const float4*)(M + (int64_t)i * n_in + 4 * c);
      const float zi = z[i];
      s.x += m.x * zi; s.y += m.y * zi; s.z += m.z * zi; s.w += m.w * zi;
    }
    *(float4*)(red + (g * cg + c) * 4) = s;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n_in; j += kBT) {
    float t = 0.f;
    for (int gg = 0; gg < rg; ++gg) t += red[(gg * cg + j / 4) * 4 + (j & 3)];
    out[j] = t + (add ? add_scale * add[j] : 0.f);
  }
  __syncthreads();
}

__device__ __forceinline__ float io_load(const void* base, int io, int64_t i) {
  if (io == TM_IO_BF16) {
    const unsigned short u = ((const unsigned short*)base)[i];
    return __uint_as_float((unsigned)u << 16);
  }
  return ((const float*)base)[i];
}


// Recompute chunk c from its checkpoint: per token j the key-side vectors at
// W_c (z, delta, b into tv), and S_t, W_t into cs[j], cw[j].  Leaves xk
// holding the last token's key.  Ends with a barrier.
__device__ void run_chunk(const BwdParams& p, int s, int c, float* base, float* lds) {
  const int64_t P = p.P;
  const int c0 = c * p.chunk;
  const int n = min(p.chunk, p.N - c0);
  const float* Wc = base + (int64_t)c * 2 * P;
  const float* Sc = Wc + P;
  float* xk = lds;                       // a_0 = k_t
  float* za = xk + p.maxw;               // z at W_c (sum of widths)
  float* aa = za + p.sumn;               // activations a_l, l = 1..L-1 (same offsets as z)
  float* dl = aa + p.sumn;               // delta
  float* bb = dl + p.sumn;               // b_l = W_{l+1}^T delta_{l+1}
  float* red = bb + p.sumn;              // kBT * 4
  const int64_t tok0 = (int64_t)s * p.N + c0;
  for (int j = 0; j < n; ++j) {
    const int64_t tt = tok0 + j;
    for (int i = threadIdx.x; i < p.d; i += kBT) xk[i] = io_load(p.k, p.io, tt * p.d + i);
    __syncthreads();
    // forward at W_c
    for (int l = 1; l <= p.L; ++l) {
      const float* ain = l == 1 ? xk : aa + p.zo[l - 1];
      mv_rows(za + p.zo[l], Wc + p.off[l], ain, p.w[l], p.w[l - 1]);
      if (l < p.L)
        for (int i = threadIdx.x; i < p.w[l]; i += kBT) aa[p.zo[l] + i] = act(za[p.zo[l] + i]);
      __syncthreads();
    }
    // backprop of 0.5 ||o - v||^2 at W_c
    for (int i = threadIdx.x; i < p.d; i += kBT) dl[p.zo[p.L] + i] = za[p.zo[p.L] + i] - io_load(p.v, p.io, tt * p.d + i);
    __syncthreads();
    for (int l = p.L; l >= 2; --l) {
      mv_cols(bb + p.zo[l - 1], Wc + p.off[l], dl + p.zo[l], p.w[l], p.w[l - 1], red);
      for (int i = threadIdx.x; i < p.w[l - 1]; i += kBT)
        dl[p.zo[l - 1] + i] = bb[p.zo[l - 1] + i] * dact(za[p.zo[l - 1] + i]);
      __syncthreads();
    }
    // key-side vectors of this token
    float* tv = base + p.o_tv + (int64_t)j * 3 * p.sumn;
    for (int i = threadIdx.x; i < p.sumn; i += kBT) {
      tv[i] = za[i];
      tv[p.sumn + i] = dl[i];
      tv[2 * p.sumn + i] = bb[i];
    }
    // S_t = eta S_{t-1} - theta delta a^T, W_t = (1 - alpha) W_{t-1} + S_t
    const int64_t gi = p.chunk_gates ? (int64_t)s * p.nchunks + c : tt;
    const float al = p.alpha[gi], et = p.eta[gi], th = p.theta[gi];
    const float* Wp = j == 0 ? Wc : base + p.o_cw + (int64_t)(j - 1) * P;
    const float* Sp = j == 0 ? Sc : base + p.o_cs + (int64_t)(j - 1) * P;
    float* Wt = base + p.o_cw + (int64_t)j * P;
    float* St = base + p.o_cs + (int64_t)j * P;
    for (int l = 1; l <= p.L; ++l) {
      const float* ain = l == 1 ? xk : aa + p.zo[l - 1];
      const float* dd = dl + p.zo[l];
      const int n_in = p.w[l - 1];
      const int64_t n4 = (int64_t)p.w[l] * n_in / 4;
#pragma unroll 4
      for (int64_t e = threadIdx.x; e < n4; e += kBT) {
        const int64_t f = p.off[l] + 4 * e;
        const int i = (int)(4 * e / n_in), m = (int)(4 * e - (int64_t)i * n_in);
        const float4 sp = *(const float4*)(Sp + f), wp = *(const float4*)(Wp + f);
        const float td = th * dd[i];
        float4 sn, wn;
        sn.x = et * sp.x - td * ain[m];     wn.x = (1.f - al) * wp.x + sn.x;
        sn.y = et * sp.y - td * ain[m + 1]; wn.y = (1.f - al) * wp.y + sn.y;
        sn.z = et * sp.z - td * ain[m + 2]; wn.z = (1.f - al) * wp.z + sn.z;
        sn.w = et * sp.w - td * ain[m + 3]; wn.w = (1.f - al) * wp.w + sn.w;
        *(float4*)(St + f) = sn;
        *(float4*)(Wt + f) = wn;
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kBT) backward_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int s = blockIdx.x;
  if (s >= p.streams) return;
  const int64_t P = p.P;
  float* base = p.ws + (int64_t)s * p.ws_stream;
  float* Wb = base + p.o_wb;
  float* Sb = base + p.o_sb;
  float* Wcb = base + p.o_wcb;

  // (W, S) at every chunk start are in the workspace: the chunked forward
  // sweep that precedes this kernel on the stream wrote them.
  // ---- reverse sweep ----
  for (int64_t e = threadIdx.x; e < P; e += kBT) {
    Wb[e] = p.dW_out ? p.dW_out[(int64_t)s * P + e] : 0.f;
    Sb[e] = p.dS_out ? p.dS_out[(int64_t)s * P + e] : 0.f;
  }
  __syncthreads();
  // LDS beyond run_chunk's area
  float* xk = lds;
  float* za = xk + p.maxw;
  float* aa = za + p.sumn;
  float* dl = aa + p.sumn;
  float* bb = dl + p.sumn;
  float* red = bb + p.sumn;            // kBT * 4
  float* xq = red + kBT * 4;           // q_t
  float* qz = xq + p.maxw;             // z of the query forward
  float* qa = qz + p.sumn;             // its activations
  float* v1 = qa + p.sumn;             // working vectors (maxw each)
  float* v2 = v1 + p.maxw;
  float* up = v2 + p.maxw;             // u'_l = Sbar_l a_{l-1} (sum of widths)
  float* db = up + p.sumn;             // deltabar
  float* zb = db + p.sumn;             // zbar
  float* zs = zb + p.sumn;             // the s'' part of zbar
  float* rp = zs + p.sumn;             // r'_l = Sbar_l^T delta_l, [L][maxw]
  float* dzq = rp + p.L * p.maxw;      // the retrieval backprop's dz_l (sum of widths)
  float* ee = dzq + p.sumn;            // e_l = deltabar_l * s'(z_l) of the Hessian-vector term

  float eta_prev = 1.f;   // Sbar still owes this factor (the last processed token's eta)
  for (int c = p.nchunks - 1; c >= 0; --c) {
    run_chunk(p, s, c, base, lds);
    const int c0 = c * p.chunk;
    const int n = min(p.chunk, p.N - c0);
    const float* Wc = base + (int64_t)c * 2 * P;
    const float* Sc = Wc + P;
    for (int64_t e = threadIdx.x; e < P; e += kBT) Wcb[e] = 0.f;
    __syncthreads();
    float gsum_a = 0.f, gsum_e = 0.f, gsum_t = 0.f;   // chunk-gate sums (thread 0)
    for (int j = n - 1; j >= 0; --j) {
      const int64_t tt = (int64_t)s * p.N + c0 + j;
      const float* Wt = base + p.o_cw + (int64_t)j * P;
      const float* Wp = j == 0 ? Wc : base + p.o_cw + (int64_t)(j - 1) * P;
      const float* Sp = j == 0 ? Sc : base + p.o_cs + (int64_t)(j - 1) * P;
      const int64_t gi = p.chunk_gates ? (int64_t)s * p.nchunks + c : tt;
      const float al = p.alpha[gi], et = p.eta[gi], th = p.theta[gi];

      // (1) retrieval: y_t = M_{Wr}(q_t)
      const float* Wr = p.read_mode == TM_READ_CHUNK_START ? Wc : Wt;
      if (p.dy) {
        for (int i = threadIdx.x; i < p.d; i += kBT) {
          xq[i] = io_load(p.q, p.io, tt * p.d + i);
          v1[i] = p.dy[tt * p.d + i];                // dz_L
        }
        __syncthreads();
        for (int l = 1; l <= p.L; ++l) {
          const float* ain = l == 1 ? xq : qa + p.zo[l - 1];
          mv_rows(qz + p.zo[l], Wr + p.off[l], ain, p.w[l], p.w[l - 1]);
          if (l < p.L)
            for (int i = threadIdx.x; i < p.w[l]; i += kBT) qa[p.zo[l] + i] = act(qz[p.zo[l] + i]);
          __syncthreads();
        }
        for (int l = p.L; l >= 1; --l) {
          // da = Wr_l^T dz_l; dz_l is kept for the fused state-adjoint passes
          mv_cols(v2, Wr + p.off[l], v1, p.w[l], p.w[l - 1], red);
          for (int i = threadIdx.x; i < p.w[l]; i += kBT) dzq[p.zo[l] + i] = v1[i];
          __syncthreads();
          if (l > 1) {
            for (int i = threadIdx.x; i < p.w[l - 1]; i += kBT) v1[i] = v2[i] * dact(qz[p.zo[l - 1] + i]);
          } else {
            for (int i = threadIdx.x; i < p.d; i += kBT) p.dq[tt * p.d + i] = v2[i];
          }
          __syncthreads();
        }
      } else {
        for (int i = threadIdx.x; i < p.d; i += kBT) p.dq[tt * p.d + i] = 0.f;
      }
      // the retrieval's rank-1 terms go to Wbar (read-after-write) or to W_c's
      // adjoint (chunk-start read); none without dL/dy (xq and qa are then unset)
      const bool rw = p.dy && p.read_mode != TM_READ_CHUNK_START;
      const bool rc = p.dy && p.read_mode == TM_READ_CHUNK_START;

      // (2) W_t = (1 - alpha) W_{t-1} + S_t, and eta's inner product.  Folded
      // into the same pass: the retrieval's rank-1 terms dz_l aq_{l-1}^T
      // (read-after-write) and the previous token's Sbar <- eta Sbar.
      float pa = 0.f, pe = 0.f;
      for (int l = 1; l <= p.L; ++l) {
        const float* aq = l == 1 ? xq : qa + p.zo[l - 1];
        const float* dz = dzq + p.zo[l];
        const int n_in = p.w[l - 1];
        const int64_t n4 = (int64_t)p.w[l] * n_in / 4;
        float4* wb4 = (float4*)(Wb + p.off[l]);
        float4* sb4 = (float4*)(Sb + p.off[l]);
        const float4* wp4 = (const float4*)(Wp + p.off[l]);
        const float4* sp4 = (const float4*)(Sp + p.off[l]);
#pragma unroll 4
        for (int64_t e = threadIdx.x; e < n4; e += kBT) {
          const int i = (int)(4 * e / n_in), j = (int)(4 * e - (int64_t)i * n_in);
          float4 wb = wb4[e], sb = sb4[e];
          const float4 wp = wp4[e], sp = sp4[e];
          if (rw) {
            const float di = dz[i];
            wb.x += di * aq[j]; wb.y += di * aq[j + 1]; wb.z += di * aq[j + 2]; wb.w += di * aq[j + 3];
          }
          pa += wb.x * wp.x + wb.y * wp.y + wb.z * wp.z + wb.w * wp.w;
          sb.x = eta_prev * sb.x + wb.x; sb.y = eta_prev * sb.y + wb.y;
          sb.z = eta_prev * sb.z + wb.z; sb.w = eta_prev * sb.w + wb.w;
          pe += sb.x * sp.x + sb.y * sp.y + sb.z * sp.z + sb.w * sp.w;
          wb.x *= 1.f - al; wb.y *= 1.f - al; wb.z *= 1.f - al; wb.w *= 1.f - al;
          wb4[e] = wb;
          sb4[e] = sb;
        }
      }
      const float abar = -block_sum(pa, red);
      const float ebar = block_sum(pe, red);

      // (3) S_t = eta S_{t-1} - theta g_t: thetabar and the Hessian-vector term at W_c
      const float* tv = base + p.o_tv + (int64_t)j * 3 * p.sumn;
      for (int i = threadIdx.x; i < p.sumn; i += kBT) {
        za[i] = tv[i];
        dl[i] = tv[p.sumn + i];
        bb[i] = tv[2 * p.sumn + i];
      }
      for (int i = threadIdx.x; i < p.d; i += kBT) xk[i] = io_load(p.k, p.io, tt * p.d + i);
      __syncthreads();
      for (int l = 1; l < p.L; ++l)
        for (int i = threadIdx.x; i < p.w[l]; i += kBT) aa[p.zo[l] + i] = act(za[p.zo[l] + i]);
      __syncthreads();
      for (int l = 1; l <= p.L; ++l) {
        const float* ain = l == 1 ? xk : aa + p.zo[l - 1];
        mv_rows(up + p.zo[l], Sb + p.off[l], ain, p.w[l], p.w[l - 1]);
        mv_cols(rp + (l - 1) * p.maxw, Sb + p.off[l], dl + p.zo[l], p.w[l], p.w[l - 1], red);
      }
      float pt = 0.f;
      for (int i = threadIdx.x; i < p.sumn; i += kBT) pt += dl[i] * up[i];
      const float tbar = -block_sum(pt, red);
      // deltabar chain, bottom-up (u = -theta u')
      for (int i = threadIdx.x; i < p.w[1]; i += kBT) db[p.zo[1] + i] = -th * up[p.zo[1] + i];
      __syncthreads();
      for (int l = 2; l <= p.L; ++l) {
        const int nl = p.w[l - 1];
        for (int i = threadIdx.x; i < nl; i += kBT) {
          const float z = za[p.zo[l - 1] + i], dbv = db[p.zo[l - 1] + i];
          ee[p.zo[l - 1] + i] = dbv * dact(z);                     // e_{l-1}
          zs[p.zo[l - 1] + i] = dbv * bb[p.zo[l - 1] + i] * d2act(z);
        }
        __syncthreads();
        mv_rows(v2, Wc + p.off[l], ee + p.zo[l - 1], p.w[l], nl);  // W_l e_{l-1}
        for (int i = threadIdx.x; i < p.w[l]; i += kBT) db[p.zo[l] + i] = -th * up[p.zo[l] + i] + v2[i];
        __syncthreads();
      }
      // v enters through delta_L = o - v; then the forward's adjoints top-down
      for (int i = threadIdx.x; i < p.d; i += kBT) {
        p.dv[tt * p.d + i] = -db[p.zo[p.L] + i];
        zb[p.zo[p.L] + i] = db[p.zo[p.L] + i];
      }
      __syncthreads();
      for (int l = p.L; l >= 1; --l) {
        const float* ain = l == 1 ? xk : aa + p.zo[l - 1];
        // abar_{l-1} = W_l^T zbar_l + r_l, r_l = -theta r'_l
        mv_cols(v2, Wc + p.off[l], zb + p.zo[l], p.w[l], p.w[l - 1], red, rp + (l - 1) * p.maxw, -th);
        // W_c's adjoint, layer l: zbar_l a_{l-1}^T + delta_l e_{l-1}^T (l >= 2), and with the
        // chunk-start read the retrieval's dz_l aq_{l-1}^T
        {
          const float* zbl = zb + p.zo[l];
          const float* dll = dl + p.zo[l];
          const float* eel = ee + p.zo[l - 1];
          const float* dzl = dzq + p.zo[l];
          const float* aq = l == 1 ? xq : qa + p.zo[l - 1];
          const bool two = l >= 2, three = rc;
          const int n_in = p.w[l - 1];
          const int64_t n4 = (int64_t)p.w[l] * n_in / 4;
          float4* m4 = (float4*)(Wcb + p.off[l]);
#pragma unroll 4
          for (int64_t e = threadIdx.x; e < n4; e += kBT) {
            const int i = (int)(4 * e / n_in), j = (int)(4 * e - (int64_t)i * n_in);
            float4 m = m4[e];
            const float zi = zbl[i];
            m.x += zi * ain[j]; m.y += zi * ain[j + 1]; m.z += zi * ain[j + 2]; m.w += zi * ain[j + 3];
            if (two) {
              const float di = dll[i];
              m.x += di * eel[j]; m.y += di * eel[j + 1]; m.z += di * eel[j + 2]; m.w += di * eel[j + 3];
            }
            if (three) {
              const float qi = dzl[i];
              m.x += qi * aq[j]; m.y += qi * aq[j + 1]; m.z += qi * aq[j + 2]; m.w += qi * aq[j + 3];
            }
            m4[e] = m;
          }
        }
        __syncthreads();
        if (l > 1) {
          for (int i = threadIdx.x; i < p.w[l - 1]; i += kBT)
            zb[p.zo[l - 1] + i] = v2[i] * dact(za[p.zo[l - 1] + i]) + zs[p.zo[l - 1] + i];
        } else {
          for (int i = threadIdx.x; i < p.d; i += kBT) p.dk[tt * p.d + i] = v2[i];
        }
        __syncthreads();
      }
      // S_{t-1}'s adjoint is eta_t Sbar: applied in the next token's pass (or at the end)
      eta_prev = et;
      if (threadIdx.x == 0) {
        if (p.chunk_gates) {
          gsum_a += abar; gsum_e += ebar; gsum_t += tbar;
        } else {
          p.dalpha[tt] = abar; p.deta[tt] = ebar; p.dtheta[tt] = tbar;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0 && p.chunk_gates) {
      const int64_t gi = (int64_t)s * p.nchunks + c;
      p.dalpha[gi] = gsum_a; p.deta[gi] = gsum_e; p.dtheta[gi] = gsum_t;
    }
    // the chunk-start state is also the previous chunk's last state
    for (int64_t e = threadIdx.x; e < P; e += kBT) Wb[e] += Wcb[e];
    __syncthreads();
  }
  for (int64_t e = threadIdx.x; e < P; e += kBT) {
    p.dW_in[(int64_t)s * P + e] = Wb[e];
    p.dS_in[(int64_t)s * P + e] = eta_prev * Sb[e];
  }
}

}  // namespace

bool backward_supported(const Shape& s, int chunk) {
  if (chunk < 1 || s.N < 1) return false;
  if (s.maxw > kMaxWidthBackward) return false;
  for (int l = 0; l <= s.L; ++l)
    if (s.widths[l] % 4 != 0) return false;
  return backward_lds_bytes(s) <= 160 * 1024;
}

int backward_lds_bytes(const Shape& s) {
  int sumn = 0;
  for (int l = 1; l <= s.L; ++l) sumn += s.widths[l];
  // run_chunk: xk, z, a, delta, b, red; reverse sweep: xq, qz, qa, v1, v2, up, db, zb, zs, rp, dzq, ee
  const int floats = s.maxw + 4 * sumn + kBT * 4 + 3 * s.maxw + 8 * sumn + s.L * s.maxw;
  return floats * 4;
}

int64_t backward_ws_floats_per_stream(const Shape& s, int chunk) {
  const int nchunks = (s.N + chunk - 1) / chunk;
  const int b = chunk < s.N ? chunk : s.N;
  int sumn = 0;
  for (int l = 1; l <= s.L; ++l) sumn += s.widths[l];
  return (int64_t)nchunks * 2 * s.P + 2 * (int64_t)b * s.P + (int64_t)b * 3 * sumn + 3 * s.P +
         (generic_ws_floats_per_stream(s, b) + 3) / 4 * 4 + 64;
}

hipError_t launch_backward(const Shape& s, int chunk, const void* k, const void* v, const void* q,
                           const float* alpha, const float* eta, const float* theta, const float* W_in,
                           const float* S_in, const float* dy, const float* dW_out, const float* dS_out, float* dk,
                           float* dv, float* dq, float* dalpha, float* deta, float* dtheta, float* dW_in,
                           float* dS_in, float* ws, hipStream_t stream) {
  BwdParams p;
  p.N = s.N;
  p.chunk = chunk;
  p.nchunks = (s.N + chunk - 1) / chunk;
  p.streams = s.streams;
  p.L = s.L;
  p.d = s.d;
  p.io = s.io;
  p.read_mode = s.read_mode;
  p.chunk_gates = s.chunk_gates;
  for (int l = 0; l <= s.L; ++l) p.w[l] = s.widths[l];
  for (int l = 1; l <= s.L; ++l) p.off[l] = s.off[l];
  p.P = s.P;
  p.maxw = s.maxw;
  int zo = 0;
  for (int l = 1; l <= s.L; ++l) {
    p.zo[l] = zo;
    zo += s.widths[l];
  }
  p.sumn = zo;
  p.zo[0] = 0;
  p.k = k; p.v = v; p.q = q;
  p.alpha = alpha; p.eta = eta; p.theta = theta;
  p.W_in = W_in; p.S_in = S_in;
  p.dy = dy; p.dW_out = dW_out; p.dS_out = dS_out;
  p.dk = dk; p.dv = dv; p.dq = dq;
  p.dalpha = dalpha; p.deta = deta; p.dtheta = dtheta;
  p.dW_in = dW_in; p.dS_in = dS_in;
  p.ws = ws;
  p.ws_stream = backward_ws_floats_per_stream(s, chunk);
  const int b = chunk < s.N ? chunk : s.N;
  p.o_cw = (int64_t)p.nchunks * 2 * s.P;
  p.o_cs = p.o_cw + (int64_t)b * s.P;
  p.o_tv = p.o_cs + (int64_t)b * s.P;
  p.o_wb = p.o_tv + ((int64_t)b * 3 * p.sumn + 3) / 4 * 4;
  p.o_sb = p.o_wb + s.P;
  p.o_wcb = p.o_sb + s.P;
  const int64_t o_gen = p.o_wcb + s.P;
  // forward sweep: the chunk-start states, through the generic kernel's
  // chunked form (its running state lives in this stream's Wbar, Sbar slots,
  // which the reverse sweep then initialises)
  hipError_t err = launch_generic_checkpoints(s, chunk, k, v, q, alpha, eta, theta, W_in, S_in, ws + p.o_wb,
                                              ws + p.o_sb, p.ws_stream, ws, p.ws_stream, ws + o_gen, p.ws_stream,
                                              stream);
  if (err != hipSuccess) return err;
  const int lds = backward_lds_bytes(s);
  p.lds_floats = lds / 4;
  err = hipFuncSetAttribute((const void*)backward_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(backward_kernel, dim3(s.streams), dim3(kBT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace titans
