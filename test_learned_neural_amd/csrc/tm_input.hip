// Input side of the memory: model activations x -> k, v, q and the gates
// alpha, eta, theta, as one bf16 MFMA GEMM per (token tile, channel tile)
// with the per-token work fused into its epilogue.
//
// What is computed ("Titans: Learning to Memorize at Test Time", mer.dev
// notes): the projections k = x W_K, v = x W_V (section 3.1, "Objective")
// and q = x W_Q (section 3.1, "Retrieving a Memory"); a causal depthwise
// 1-D convolution over time after each projection (section 4.4,
// "Convolution"); SiLU on all three and an l2 normalisation of k and q over
// each head's channels (section 4.4, "Architectural Details"); and
// input-dependent gates (section 3.1, "Learning Process and Surprise
// Metric"), here scale * sigmoid(x . w + b) per head and gate.
//
// Mapping on gfx950:
// - The GEMM is [B*N tokens x D] . [D x (3*H*d + 3*H) channels].  A
//   workgroup (4 waves) computes 256 consecutive token rows x 128 channels
//   and writes the last 256 - (w-1) of them: the first w-1 rows are the
//   convolution's halo, recomputed instead of exchanged (1.2% extra work
//   at w = 4).  Rows of different sequences may share a tile; a tap that
//   would reach before its sequence's start is dropped.
// - Operands go global -> LDS with global_load_lds (no registers), two
//   stages of 32-deep slices, each 16-byte chunk of a 64-byte row slice
//   stored at chunk ^ ((row >> 1) & 3) so that the fragment reads of eight
//   consecutive rows hit eight different 16-byte bank groups.
// - Each wave owns 64 token rows x 128 channels: 2 x 4 accumulators of
//   v_mfma_f32_32x32x16_bf16 (128 fp32 per lane).  bf16 x bf16 products are
//   exact in fp32; sums are fp32.
// - Epilogue: the fp32 tile goes through LDS, one pass of max(64, d)
//   channels at a time; groups of d/4 lanes own one (token, head) with 4
//   channels per lane for the convolution, SiLU, the head's sum of squares
//   (lane shuffles), the normalisation and the bf16 store (8 bytes per lane,
//   a head row per group).  Gate tiles read logits from a padded LDS copy
//   with one thread per token, so stores of a gate row are contiguous.
// - Grid: block i runs on XCD i % 8 (round-robin dispatch); blocks of one
//   XCD take its token tiles in turn and sweep all channel tiles of each,
//   so the 512 KiB x tile is reused from that XCD's L2.
#include "tm_internal.h"

namespace titans {
namespace {

constexpr int kMT = 256;          // token rows computed per tile
constexpr int kNT = 128;          // channels per tile
constexpr int kKT = 32;           // reduction depth per stage
constexpr int kThreads = 256;
constexpr int kStageA = kMT * kKT * 2;
constexpr int kStageB = kNT * kKT * 2;
constexpr int kStage = kStageA + kStageB;
constexpr int kGatePass = 64;     // gate logits per epilogue pass
constexpr int kGateStride = kGatePass + 1;
constexpr float kNormFloor2 = 1e-12f;   // (1e-6)^2: k, q = s / max(||s||, 1e-6)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

struct InParams {
  const uint16_t* x;      // [R, D] bf16, R = B * N
  const uint16_t* wp;     // [3C, D] bf16: rows of W_K, W_V, W_Q
  const float* conv;      // [3C, w]
  const uint16_t* wg;     // [3H, D] bf16
  const float* bg;        // [3H]
  float scale[3];
  uint16_t* kvq[3];       // [B, H, N, d] bf16
  float* gate[3];         // [B, H, N]
  int64_t R;
  int64_t n_row_tiles;
  int N, D, H, C, w, halo, mo;
  int n_kvq_tiles, n_col_tiles;
};

template <int kD>
constexpr int pass_width() { return kD > 64 ? kD : 64; }

template <int kD>
constexpr int lds_bytes() {
  int m = 2 * kStage;
  if (kMT * pass_width<kD>() * 4 > m) m = kMT * pass_width<kD>() * 4;
  if (kMT * kGateStride * 4 > m) m = kMT * kGateStride * 4;
  return m;
}

__device__ __forceinline__ float sigmoidf(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Stage `stage` <- x rows [r0, r0 + 256) and weight rows [0, 128) of
// columns [k0, k0 + 32).  Each instruction fills 16 rows (1 KiB); lane l
// writes row 16 g + l / 4, chunk slot l % 4, which holds source chunk
// (l % 4) ^ ((row >> 1) & 3).  Rows outside [0, R) and weight rows past
// `wrows` load a clamped row whose results are never stored.
__device__ __forceinline__ void issue_stage(const InParams& p, unsigned char* smem, int stage, int k0,
                                            int64_t r0, const uint16_t* w0, int wrows, int wv, int lane) {
  unsigned char* sa = smem + stage * kStage;
  unsigned char* sb = sa + kStageA;
  const int sub = lane >> 2, cs = lane & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wv * 4 + i;
    const int rr = g * 16 + sub;
    const int c = cs ^ ((rr >> 1) & 3);
    int64_t gr = r0 + rr;
    gr = gr < 0 ? 0 : (gr >= p.R ? p.R - 1 : gr);
    __builtin_amdgcn_global_load_lds((const void*)(p.x + gr * p.D + k0 + c * 8), (lds_void_ptr)(sa + g * 1024),
                                     16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = wv * 2 + i;
    const int rr = g * 16 + sub;
    const int c = cs ^ ((rr >> 1) & 3);
    const int wr = rr < wrows ? rr : wrows - 1;
    __builtin_amdgcn_global_load_lds((const void*)(w0 + (int64_t)wr * p.D + k0 + c * 8),
                                     (lds_void_ptr)(sb + g * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 frag(const unsigned char* base, int row, int c) {
  return *(const bf16x8*)(base + row * 64 + 16 * (c ^ ((row >> 1) & 3)));
}

// accumulator register r of a 32x32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int kD>
__device__ __forceinline__ void kvq_epilogue(const InParams& p, float* ep, const f32x16 (&acc)[2][4], int col,
                                             int64_t r0, int tid) {
  constexpr int PW = pass_width<kD>();
  constexpr int G = kD / 4;          // lanes per (token, head)
  constexpr int HP = PW / kD;        // heads per pass
  constexpr int NR = kThreads / G / HP;   // token ranges per pass
  const int lane = tid & 63, wv = tid >> 6;
  const int gid = tid / G, sl = tid % G;
  const int hp = gid % HP, rg = gid / HP;
  const int rpr = (p.mo + NR - 1) / NR;
  const int i0 = p.halo + rg * rpr;
  const int i1 = i0 + rpr < kMT ? i0 + rpr : kMT;
#pragma unroll
  for (int pp = 0; pp < kNT / PW; ++pp) {
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = pp * PW / 32; ct < (pp + 1) * PW / 32; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(64 * wv + 32 * rt + acc_row(r, lane)) * PW + 32 * ct - pp * PW + (lane & 31)] = acc[rt][ct][r];
    __syncthreads();

    const int cl = hp * kD + 4 * sl;                 // channel within the pass
    const int cg = col * kNT + pp * PW + cl;         // channel in [0, 3C)
    const int which = cg / p.C;
    const int hc = cg - which * p.C;
    const int h = hc / kD, cq = hc - h * kD;
    float tap[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) tap[j][tau] = tau < p.w ? p.conv[(int64_t)(cg + j) * p.w + tau] : 0.0f;
    if (i0 >= i1) continue;
    int64_t gr = r0 + i0;
    if (gr >= p.R) continue;
    int64_t bb = gr / p.N;
    int t = (int)(gr - bb * p.N);
    uint16_t* out = p.kvq[which];
    for (int i = i0; i < i1; ++i, ++gr) {
      if (gr >= p.R) break;
      float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) {
        if (tau < p.w && tau <= t) {
          const float4 pv = *(const float4*)(ep + (i - tau) * PW + cl);
          u[0] += tap[0][tau] * pv.x;
          u[1] += tap[1][tau] * pv.y;
          u[2] += tap[2][tau] * pv.z;
          u[3] += tap[3][tau] * pv.w;
        }
      }
      float s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = u[j] * sigmoidf(u[j]);
      if (which != 1) {
        float ss = s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3];
#pragma unroll
        for (int m = 1; m < G; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = __builtin_amdgcn_rsqf(ss > kNormFloor2 ? ss : kNormFloor2);
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] *= inv;
      }
      uint2 pk;
      pk.x = pack_bf16(s[0], s[1]);
      pk.y = pack_bf16(s[2], s[3]);
      *(uint2*)(out + ((bb * p.H + h) * p.N + t) * kD + cq) = pk;
      if (++t == p.N) {
        t = 0;
        ++bb;
      }
    }
  }
}

__device__ __forceinline__ void gate_epilogue(const InParams& p, float* ep, const f32x16 (&acc)[2][4], int gbase,
                                              int64_t r0, int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  const int i = tid;                 // one token row per thread
  const int64_t gr = r0 + i;
  const bool live = i >= p.halo && gr < p.R;
  const int64_t bb = live ? gr / p.N : 0;
  const int t = live ? (int)(gr - bb * p.N) : 0;
#pragma unroll
  for (int pp = 0; pp < kNT / kGatePass; ++pp) {
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 2 * pp; ct < 2 * pp + 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(64 * wv + 32 * rt + acc_row(r, lane)) * kGateStride + 32 * (ct - 2 * pp) + (lane & 31)] =
              acc[rt][ct][r];
    __syncthreads();
    if (!live) continue;
    for (int c = 0; c < kGatePass; ++c) {
      const int gc = gbase + pp * kGatePass + c;
      if (gc >= 3 * p.H) break;
      const int g = gc / p.H, h = gc - g * p.H;
      const float z = ep[i * kGateStride + c] + p.bg[gc];
      const float sc = g == 0 ? p.scale[0] : (g == 1 ? p.scale[1] : p.scale[2]);
      float* dst = g == 0 ? p.gate[0] : (g == 1 ? p.gate[1] : p.gate[2]);
      dst[(bb * p.H + h) * p.N + t] = sc * sigmoidf(z);
    }
  }
}

template <int kD>
__global__ __launch_bounds__(kThreads, 2) void input_kernel(InParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bi = blockIdx.x;
  const int64_t m = bi >> 3;
  const int col = (int)(m % p.n_col_tiles);
  const int64_t rt = (bi & 7) + 8 * (m / p.n_col_tiles);
  if (rt >= p.n_row_tiles) return;
  const int64_t r0 = rt * p.mo - p.halo;
  const bool gate_tile = col >= p.n_kvq_tiles;
  const int gbase = (col - p.n_kvq_tiles) * kNT;
  const uint16_t* w0 = gate_tile ? p.wg + (int64_t)gbase * p.D : p.wp + (int64_t)col * kNT * p.D;
  const int wrows = gate_tile ? (3 * p.H - gbase < kNT ? 3 * p.H - gbase : kNT) : kNT;

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // Two-stage pipeline.  The barriers are plain s_barrier with explicit
  // waits: a __syncthreads() fence would also wait for the next stage's
  // loads.  A wave's LDS-direct loads have written LDS once its vmcnt has
  // dropped past them; the asm memory clobbers keep LDS reads in place.
  const int nk = p.D / kKT;
  issue_stage(p, smem, 0, 0, r0, w0, wrows, wv, lane);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      issue_stage(p, smem, (kt + 1) & 1, (kt + 1) * kKT, r0, w0, wrows, wv, lane);
      asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");   // this stage's six loads landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const unsigned char* sa = smem + (kt & 1) * kStage;
    const unsigned char* sb = sa + kStageA;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * s + (lane >> 5);
      bf16x8 a[2], b[4];
#pragma unroll
      for (int r = 0; r < 2; ++r) a[r] = frag(sa, 64 * wv + 32 * r + (lane & 31), c);
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = frag(sb, 32 * q + (lane & 31), c);
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[r][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[q], acc[r][q], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stage fully read before its refill
  }

  float* ep = (float*)smem;
  if (gate_tile)
    gate_epilogue(p, ep, acc, gbase, r0, tid);
  else
    kvq_epilogue<kD>(p, ep, acc, col, r0, tid);
}

template <int kD>
hipError_t launch_d(const InParams& p, int64_t grid, hipStream_t stream) {
  const int lds = lds_bytes<kD>();
  hipError_t err = hipFuncSetAttribute((const void*)input_kernel<kD>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(input_kernel<kD>, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

bool input_supported(int D, int H, int d, int w) {
  if (D <= 0 || D % kKT != 0) return false;
  if (d != 16 && d != 32 && d != 64 && d != 128) return false;
  if (H <= 0 || ((int64_t)H * d) % kNT != 0) return false;
  if ((int64_t)H * d * 3 > (1 << 28)) return false;
  return w >= 1 && w <= 4;
}

int64_t input_grid(int64_t R, int D, int H, int d, int w) {
  (void)D;
  const int mo = kMT - (w - 1);
  const int64_t rows = (R + mo - 1) / mo;
  const int64_t rows8 = (rows + 7) / 8 * 8;
  const int64_t cols = (int64_t)3 * H * d / kNT + (3 * H + kNT - 1) / kNT;
  return rows8 * cols;
}

hipError_t launch_input(int B, int N, int D, int H, int d, int w, const void* x, const void* w_proj,
                        const float* conv_w, const void* w_gate, const float* b_gate, const float scale[3],
                        void* const kvq[3], float* const gates[3], hipStream_t stream) {
  InParams p;
  p.x = (const uint16_t*)x;
  p.wp = (const uint16_t*)w_proj;
  p.conv = conv_w;
  p.wg = (const uint16_t*)w_gate;
  p.bg = b_gate;
  for (int i = 0; i < 3; ++i) {
    p.scale[i] = scale[i];
    p.kvq[i] = (uint16_t*)kvq[i];
    p.gate[i] = gates[i];
  }
  p.R = (int64_t)B * N;
  p.N = N;
  p.D = D;
  p.H = H;
  p.C = H * d;
  p.w = w;
  p.halo = w - 1;
  p.mo = kMT - p.halo;
  p.n_row_tiles = (p.R + p.mo - 1) / p.mo;
  p.n_kvq_tiles = 3 * p.C / kNT;
  p.n_col_tiles = p.n_kvq_tiles + (3 * H + kNT - 1) / kNT;
  const int64_t grid = input_grid(p.R, D, H, d, w);
  switch (d) {
    case 16: return launch_d<16>(p, grid, stream);
    case 32: return launch_d<32>(p, grid, stream);
    case 64: return launch_d<64>(p, grid, stream);
    default: return launch_d<128>(p, grid, stream);
  }
}

}  // namespace titans
