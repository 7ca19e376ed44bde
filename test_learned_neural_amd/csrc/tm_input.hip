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
//   v_mfma_f32_32x32x16_bf16 (128 fp32 per lane), computed transposed
//   (weights as the first operand: accumulator rows are channels, lanes are
//   tokens).  bf16 x bf16 products are exact in fp32; sums are fp32.
// - Epilogue: the fp32 tile goes through LDS (each lane's four consecutive
//   channels of a token as one 16-byte store, rows padded to 68 floats), one
//   pass of max(64, d) channels at a time; groups of d/4 lanes own one
//   (token, head) with 4
//   channels per lane for the convolution, SiLU, the head's sum of squares
//   (lane shuffles), the normalisation and the bf16 store (8 bytes per lane,
//   a head row per group).  Gate tiles read logits from a padded LDS copy
//   with one thread per token, so stores of a gate row are contiguous.
// - Grid: block i runs on XCD i % 8 (round-robin dispatch).  An XCD takes
//   its token tiles in groups of 8 and walks the channel tiles once per
//   group, the 8 token tiles of a group side by side: a channel tile's
//   256 KiB of weights is then fetched into the XCD's L2 once per group
//   instead of once per token tile (6.4 MiB of weights do not fit a 4 MiB
//   L2), and each 512 KiB x tile stays there while the group runs.
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
constexpr int kRowGroup = 8;      // token tiles of one XCD sharing each channel tile's weights
constexpr int kGatePass = 64;     // gate logits per epilogue pass
constexpr int kGateStride = kGatePass + 4;   // padded row (16-byte aligned rows for the tile writes)
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
// row pitch (floats) of the epilogue's fp32 tile: padded so that the
// accumulators' 16-byte row pieces of 32 consecutive rows spread over banks
template <int kD>
constexpr int ep_stride() { return pass_width<kD>() + 4; }

template <int kD>
constexpr int lds_bytes() {
  int m = 2 * kStage;
  if (kMT * ep_stride<kD>() * 4 > m) m = kMT * ep_stride<kD>() * 4;
  if (kMT * kGateStride * 4 > m) m = kMT * kGateStride * 4;
  return m;
}

__device__ __forceinline__ float sigmoidf(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// two floats -> two bf16 (nearest-even) in one register: v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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

// Sum over aligned groups of G lanes (G = 4, 8, 16, 32), result in every
// lane of the group: DPP quad permutations, then half-row and row mirrors
// (lane i meets lane 7 - i, then 15 - i, whose partial sums cover the other
// half), and a cross-row swap for 32.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);                  // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                  // quad_perm [2,3,0,1]
  if (G >= 8) x += dpp<0x141>(x);     // row_half_mirror
  if (G >= 16) x += dpp<0x140>(x);    // row_mirror
  if (G >= 32) x += __shfl_xor(x, 16);
  return x;
}

// accumulator register r of a 32x32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int kD>
__device__ __forceinline__ void kvq_epilogue(const InParams& p, float* ep, const f32x16 (&acc)[2][4], int col,
                                             int64_t r0, int tid) {
  constexpr int PW = pass_width<kD>();
  constexpr int ES = ep_stride<kD>();
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
        for (int g = 0; g < 4; ++g)   // registers 4g .. 4g+3: channels acc_row(4g, lane) .. +3 of token lane % 32
          *(float4*)(ep + (64 * wv + 32 * rt + (lane & 31)) * ES + 32 * ct - pp * PW + acc_row(4 * g, lane)) =
              make_float4(acc[rt][ct][4 * g], acc[rt][ct][4 * g + 1], acc[rt][ct][4 * g + 2], acc[rt][ct][4 * g + 3]);
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
    // rows [i0, iend) of this range; rows past the last token are not stored
    const int iend = (int)(r0 + i1 <= p.R ? i1 : p.R - r0);
    if (i0 >= iend) continue;
    const int64_t gr0 = r0 + i0;
    int64_t bb = gr0 / p.N;
    int t = (int)(gr0 - bb * p.N);
    uint16_t* base = p.kvq[which];
    uint16_t* dst = base + ((bb * p.H + h) * p.N + t) * kD + cq;
    // the three previous rows' projections (rows before the tile's halo
    // are never needed: i0 - tau < 0 only for taps tau >= w, which are 0)
    float4 w1 = p.w > 1 ? *(const float4*)(ep + (i0 - 1) * ES + cl) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 w2 = p.w > 2 ? *(const float4*)(ep + (i0 - 2) * ES + cl) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 w3 = p.w > 3 ? *(const float4*)(ep + (i0 - 3) * ES + cl) : make_float4(0.f, 0.f, 0.f, 0.f);
    auto emit = [&](const float4& c, const float4& a1, const float4& a2, const float4& a3, uint16_t* o) {
      const float u0 = tap[0][0] * c.x + tap[0][1] * a1.x + tap[0][2] * a2.x + tap[0][3] * a3.x;
      const float u1 = tap[1][0] * c.y + tap[1][1] * a1.y + tap[1][2] * a2.y + tap[1][3] * a3.y;
      const float u2 = tap[2][0] * c.z + tap[2][1] * a1.z + tap[2][2] * a2.z + tap[2][3] * a3.z;
      const float u3 = tap[3][0] * c.w + tap[3][1] * a1.w + tap[3][2] * a2.w + tap[3][3] * a3.w;
      float s0 = u0 * sigmoidf(u0), s1 = u1 * sigmoidf(u1), s2 = u2 * sigmoidf(u2), s3 = u3 * sigmoidf(u3);
      if (which != 1) {
        const float ss = group_sum<G>(s0 * s0 + s1 * s1 + s2 * s2 + s3 * s3);
        const float inv = __builtin_amdgcn_rsqf(ss > kNormFloor2 ? ss : kNormFloor2);
        s0 *= inv;
        s1 *= inv;
        s2 *= inv;
        s3 *= inv;
      }
      uint2 pk;
      pk.x = pack_bf16(s0, s1);
      pk.y = pack_bf16(s2, s3);
      *(uint2*)o = pk;
    };
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t >= 3 && t + (iend - i0) <= p.N) {
      // no sequence start in the range: every tap is live, the output row
      // advances by one head row per token
      int i = i0;
      for (; i + 4 <= iend; i += 4) {
        const float4 c0 = *(const float4*)(ep + (i + 0) * ES + cl);
        const float4 c1 = *(const float4*)(ep + (i + 1) * ES + cl);
        const float4 c2 = *(const float4*)(ep + (i + 2) * ES + cl);
        const float4 c3 = *(const float4*)(ep + (i + 3) * ES + cl);
        emit(c0, w1, w2, w3, dst);
        emit(c1, c0, w1, w2, dst + kD);
        emit(c2, c1, c0, w1, dst + 2 * kD);
        emit(c3, c2, c1, c0, dst + 3 * kD);
        dst += 4 * kD;
        w3 = c1;
        w2 = c2;
        w1 = c3;
      }
      for (; i < iend; ++i) {
        const float4 c0 = *(const float4*)(ep + i * ES + cl);
        emit(c0, w1, w2, w3, dst);
        dst += kD;
        w3 = w2;
        w2 = w1;
        w1 = c0;
      }
    } else {
      // a sequence starts inside the range (or just before it): taps that
      // would reach before the start are dropped
      for (int i = i0; i < iend; ++i) {
        const float4 c0 = *(const float4*)(ep + i * ES + cl);
        emit(c0, t >= 1 ? w1 : z4, t >= 2 ? w2 : z4, t >= 3 ? w3 : z4, dst);
        w3 = w2;
        w2 = w1;
        w1 = c0;
        if (++t == p.N) {
          t = 0;
          ++bb;
          dst = base + (bb * p.H + h) * (int64_t)p.N * kD + cq;
        } else {
          dst += kD;
        }
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
        for (int g = 0; g < 4; ++g)
          *(float4*)(ep + (64 * wv + 32 * rt + (lane & 31)) * kGateStride + 32 * (ct - 2 * pp) + acc_row(4 * g, lane)) =
              make_float4(acc[rt][ct][4 * g], acc[rt][ct][4 * g + 1], acc[rt][ct][4 * g + 2], acc[rt][ct][4 * g + 3]);
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
  const int64_t m = bi >> 3;                    // position in this XCD's sequence
  const int64_t grp = m / (kRowGroup * p.n_col_tiles);
  const int idx = (int)(m - grp * (kRowGroup * p.n_col_tiles));
  const int col = idx / kRowGroup;
  const int64_t rt = (bi & 7) + 8 * (grp * kRowGroup + idx % kRowGroup);
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
        for (int q = 0; q < 4; ++q) acc[r][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q], a[r], acc[r][q], 0, 0, 0);
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
  // token tiles padded to whole groups on every XCD; the padding exits at once
  const int mo = kMT - (w - 1);
  const int64_t rows = (R + mo - 1) / mo;
  const int64_t per_xcd = ((rows + 7) / 8 + kRowGroup - 1) / kRowGroup * kRowGroup;
  const int64_t cols = (int64_t)3 * H * d / kNT + (3 * H + kNT - 1) / kNT;
  return 8 * per_xcd * cols;
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
