// Retrieval at a fixed state on the matrix cores: y = M_W(q) for the 2-layer
// memory with d = 64 and hidden = 256, bf16 queries and outputs ("Titans:
// Learning to Memorize at Test Time", mer.dev notes, section 3.1 "Retrieving
// a Memory": a forward pass of the memory without any weight change;
// M(q) = W2 SiLU(W1 q), section 3.1 "Memory Architecture").
//
// Mapping on gfx950:
// - A workgroup (4 waves) serves 1024 consecutive tokens of one stream.  Each
//   wave converts its share of the stream's fp32 W1 [256 x 64] and W2
//   [64 x 256] (its 64 hidden units) to bf16 once (round to nearest even)
//   and keeps them in registers as ready MFMA operands (64 VGPRs); LDS holds
//   only the query tile and the partial outputs, so two workgroups share a
//   CU.
// - Per 64-token tile, wave w computes Z1^T = W1 Q^T for hidden units
//   64w .. 64w+63 with v_mfma_f32_32x32x16_bf16 (four 32x32 tiles, K = 64),
//   applies SiLU to the fp32 accumulators and feeds them, rounded to bf16,
//   straight back as the operand of y^T = W2 A1^T: an accumulator tile
//   (lane = token, registers = hidden rows) is an operand contracting over
//   its rows, in the order of its registers, so W2's fragments are read in
//   that same order (two 8-byte pieces per lane and K-step) and A1 never goes
//   through memory.
// - Each wave thus holds y over its 64 hidden units; the four partial tiles
//   are summed through LDS in a fixed order and stored as bf16, one 32-byte
//   piece of a token row per thread.
// bf16 operands keep y within a few 1e-3 of the exact value (each product
// carries two roundings of 2^-9); sums are fp32.
#include "tm_internal.h"

#include <hip/hip_bf16.h>

namespace titans {
namespace {

constexpr int kD = 64, kH = 256;
constexpr int kThreads = 256;
constexpr int kTok = 64;               // tokens per tile
constexpr int kRange = 1024;           // tokens per workgroup
constexpr int RS1 = kD + 8;            // bf16 row stride of the query tile [t][d]
constexpr int RSY = kD + 4;            // fp32 row stride of the partial y [t][c]
constexpr int OFF_Q = 0;
constexpr int OFF_Y = OFF_Q + kTok * RS1 * 2;
constexpr int kLds = OFF_Y + 4 * kTok * RSY * 4;
static_assert(2 * kLds <= 160 * 1024, "two workgroups per CU");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

struct RParams {
  const uint16_t* q;   // [S, N, 64] bf16
  const float* W;      // [S, P]
  uint16_t* y;         // [S, N, 64] bf16
  int N, ranges;       // ranges of kRange tokens per stream
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
  bf16x8 r;
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
  return r;
}

__global__ void __launch_bounds__(kThreads, 2) mlp2_retrieve_kernel(RParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* qs = (uint16_t*)(smem + OFF_Q);
  float* yp = (float*)(smem + OFF_Y);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x / p.ranges;
  const int t_begin = (blockIdx.x % p.ranges) * kRange;
  const int t_end = min(t_begin + kRange, p.N);
  if (t_begin >= t_end) return;

  // ---- this wave's weight fragments, bf16, in registers for the whole range ----
  // W1 rows 64w + 32ht + lr (the A operand of Z1^T, K = d in order);
  // W2 [c][h] for this wave's hidden units in the accumulator row order
  // (the A operand of y^T: rows 16ks + 4lg + 0..3 and 16ks + 8 + 4lg + 0..3)
  const float* W = p.W + (int64_t)s * (2 * kD * kH);
  bf16x8 w1f[2][4], w2f[2][2][2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* src = W + (64 * w + 32 * ht + lr) * kD + 16 * ks + 8 * lg;
      w1f[ht][ks] = to_bf16x8(*(const float4*)src, *(const float4*)(src + 4));
    }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float* src = W + kH * kD + (32 * ct + lr) * kH + 64 * w + 32 * ht + 16 * ks + 4 * lg;
        w2f[ct][ht][ks] = to_bf16x8(*(const float4*)src, *(const float4*)(src + 8));
      }

  const uint16_t* qst = p.q + (int64_t)s * p.N * kD;
  uint16_t* yst = p.y + (int64_t)s * p.N * kD;
  // this thread's 32 bytes of a query row (row tid / 4), loaded one tile
  // ahead; rows past the end read as zero
  const int qj = tid >> 2, qc = (tid & 3) * 16;
  auto load_q = [&](int t0, uint4& a, uint4& b) {
    a = b = make_uint4(0, 0, 0, 0);
    if (t0 + qj < t_end) {
      const uint4* src = (const uint4*)(qst + (int64_t)(t0 + qj) * kD + qc);
      a = src[0];
      b = src[1];
    }
  };
  uint4 qa, qb;
  load_q(t_begin, qa, qb);
  for (int t0 = t_begin; t0 < t_end; t0 += kTok) {
    const int n = min(kTok, t_end - t0);
    *(uint4*)(qs + qj * RS1 + qc) = qa;
    *(uint4*)(qs + qj * RS1 + qc + 8) = qb;
    __syncthreads();
    if (t0 + kTok < t_end) load_q(t0 + kTok, qa, qb);   // the next tile's rows, in flight during this one

    // ---- Z1^T = W1 Q^T for hidden rows 64w .. 64w+63 (2 x 2 tiles, K = 64) ----
    f32x16 z[2][2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) z[ht][tt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 b[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) b[tt] = *(const bf16x8*)(qs + (32 * tt + lr) * RS1 + 16 * ks + 8 * lg);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          z[ht][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1f[ht][ks], b[tt], z[ht][tt], 0, 0, 0);
    }
    // ---- A1 = SiLU(Z1), as bf16 operands contracting over the hidden rows ----
    bf16x8 a1[2][2][2];   // [ht][tt][K-step within the 32-row tile]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = z[ht][tt][r];
          a1[ht][tt][r >> 3][r & 7] = (__bf16)(x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)));
        }

    // ---- partial y^T = W2 A1^T over this wave's 64 hidden units (2 x 2 tiles) ----
    f32x16 yacc[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) yacc[ct][tt][r] = 0.f;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            yacc[ct][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2f[ct][ht][ks], a1[ht][tt][ks], yacc[ct][tt], 0, 0, 0);
    // registers 4g .. 4g+3 of tile (ct, tt): channels 32 ct + 8 g + 4 lg + 0..3 of token 32 tt + lr
    float* ypw = yp + w * kTok * RSY;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(ypw + (32 * tt + lr) * RSY + 32 * ct + 8 * g + 4 * lg) =
              make_float4(yacc[ct][tt][4 * g], yacc[ct][tt][4 * g + 1], yacc[ct][tt][4 * g + 2], yacc[ct][tt][4 * g + 3]);
    __syncthreads();

    // ---- y = sum of the four partials (fixed order), bf16 ----
    {
      const int j = tid >> 2, cb = (tid & 3) * 16;
      if (j < n) {
        float acc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int src = 0; src < 4; ++src) {
          const float* rowp = yp + src * kTok * RSY + j * RSY + cb;
#pragma unroll
          for (int i = 0; i < 16; i += 4) {
            const float4 v = *(const float4*)(rowp + i);
            acc[i] += v.x; acc[i + 1] += v.y; acc[i + 2] += v.z; acc[i + 3] += v.w;
          }
        }
        uint4* dst = (uint4*)(yst + (int64_t)(t0 + j) * kD + cb);
        dst[0] = make_uint4(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]), pack2(acc[4], acc[5]), pack2(acc[6], acc[7]));
        dst[1] = make_uint4(pack2(acc[8], acc[9]), pack2(acc[10], acc[11]), pack2(acc[12], acc[13]),
                            pack2(acc[14], acc[15]));
      }
    }
    __syncthreads();   // the next tile rewrites the query tile and the partials
  }
}

}  // namespace

bool retrieve_mlp2_supported(const Shape& s) {
  return s.L == 2 && s.d == kD && s.hidden == kH && s.io == TM_IO_BF16;
}

hipError_t launch_retrieve_mlp2(const Shape& s, const void* q, const float* W, void* y, hipStream_t stream) {
  RParams p;
  p.q = (const uint16_t*)q;
  p.W = W;
  p.y = (uint16_t*)y;
  p.N = s.N;
  p.ranges = (s.N + kRange - 1) / kRange;
  const int64_t grid = (int64_t)s.streams * p.ranges;
  if (grid <= 0) return hipSuccess;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  hipError_t e = hipFuncSetAttribute((const void*)mlp2_retrieve_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mlp2_retrieve_kernel, dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
  return hipGetLastError();
}

}  // namespace titans
