// Workgroup-wide fp32 contraction on the matrix cores, shared by the
// shape-generic forward sweep and the chunk-wise backward sweep (device code
// only; each translation unit gets its own copy).
#pragma once

#include <hip/hip_runtime.h>

namespace titans {
namespace {

constexpr int kGemmThreads = 512;   // workgroup size every caller launches with
constexpr int kGemmTile = 64;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C[M x N] = sum_k A(m, k) B(k, n), handed to an epilogue per element.  The
// whole workgroup (eight waves, two per SIMD, so one wave's memory waits
// overlap the other's work) cooperates; operands come through accessors
// (global/L2 reads) and are staged through LDS in kGk-deep slices, the next
// slice's operands loaded into registers while the current one is
// multiplied.  Output tiles are 64 x 128 when N > 64, else 64 x 64; with
// eight waves each wave of a wide tile computes one 32 x 32 block over the
// whole slice, and in a narrow tile two waves share a block, each over half
// the slice's k, the second handing its partial sums to the first through
// LDS at the end.  A wave splits its k over two accumulators, i.e. two
// independent chains of the fp32 matrix instruction v_mfma_f32_32x32x2_f32
// (lane l supplies A[l%32][l/32] and B[l/32][l%32]; accumulator register r
// holds row 8(r/4) + 4(l/32) + r%4, column l%32), summed before the
// epilogue, and the arithmetic stays fp32.  The accessors
// are read in the order that keeps a wavefront's loads on few cache lines:
// A_KMAJOR says A(m, k) is contiguous in k (else in m); bkmaj(k0) says
// whether the B slice starting at k0 is contiguous in k (else in n).
//
// So that a wave keeps all of a slice's loads in flight at once, the
// accessors and the epilogue are called unconditionally, with indices
// clamped into range (M, N, K >= 1): fa(m, k) and fb(k, n) must be
// branch-free reads of valid addresses (an accessor that selects between
// arrays keeps every arm's pointer in range, read or not: an out-of-range
// pointer is undefined and lets the compiler fold the selection wrongly);
// operands outside the product are zeroed when staged.  The epilogue is split in two: pre(m, n) reads what
// the element's update needs (any value type), epi(m, n, value, pre, ok)
// stores, only where ok is set.
constexpr int kGk = 32;                                  // k per staged slice
constexpr int kGN = 2 * kGemmTile;                       // output columns per wide tile
constexpr int kGPerA = kGemmTile * kGk / kGemmThreads;   // A elements per thread per slice
constexpr int kGPerB = kGN * kGk / kGemmThreads;         // B elements per thread per wide slice
constexpr int kEpiGroup = 8;                             // accumulator rows per epilogue group
constexpr int kGemmWaves = kGemmThreads / 64;
constexpr int kGemmStageFloats = kGk * (kGemmTile + 1) + kGk * (kGN + 1);
constexpr int kGemmRedFloats = 4 * (kGemmWaves / 4 - 1) * 64 * 17;   // narrow tiles: 4 blocks
constexpr int kGemmLdsFloats = kGemmStageFloats > kGemmRedFloats ? kGemmStageFloats : kGemmRedFloats;

// one LDS allocation shared by every block_gemm instantiation of a kernel
__device__ __forceinline__ float* gemm_lds() {
  __shared__ float buf[kGemmLdsFloats];
  return buf;
}

template <bool A_KMAJOR, bool WIDE, class FA, class FB, class FBK, class FP, class FE>
__device__ void block_gemm_tiles(int M, int N, int K, FA fa, FB fb, FBK bkmaj, FP pre, FE epi) {
  using PreT = decltype(pre(0, 0));
  float* As = gemm_lds();                   // [kGk][kGemmTile + 1]
  float* Bs = As + kGk * (kGemmTile + 1);   // [kGk][kGN + 1]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (wave-uniform)
  constexpr bool wide = WIDE;
  constexpr int tn = wide ? kGN : kGemmTile;       // output columns per tile
  constexpr int nb = wide ? kGPerB : kGPerB / 2;   // B elements per thread per slice
  // the tile's 32 x 32 blocks (8 wide, 4 narrow) are shared out over the
  // waves; the ksplit waves of one block each take 1/ksplit of the slice's k
  constexpr int nblk = wide ? 8 : 4;                 // 32 x 32 blocks per tile
  constexpr int ksplit = kGemmWaves / nblk;          // waves per block, each over part of the slice's k
  const int blk = wv / ksplit;
  const int wm = wide ? (blk >> 2) * 32 : (blk >> 1) * 32;
  const int wn = wide ? (blk & 3) * 32 : (blk & 1) * 32;
  const int kh = wv % ksplit;
  const int li = lane & 31, lk = lane >> 5;
  auto a_at = [&](int q, int& mm, int& ka) {
    const int e = tid + q * kGemmThreads;
    if (A_KMAJOR) { mm = e / kGk; ka = e % kGk; } else { ka = e / kGemmTile; mm = e % kGemmTile; }
  };
  auto b_at = [&](bool kmaj, int q, int& kb, int& nn) {
    const int e = tid + q * kGemmThreads;
    if (kmaj) { nn = e / kGk; kb = e % kGk; } else { kb = e / tn; nn = e % tn; }
  };
  // the workgroups of a launch's y dimension share out the output tiles
  // (one workgroup, gridDim.y == 1, takes them all)
  const int ntn = (N + tn - 1) / tn, ntiles = ((M + kGemmTile - 1) / kGemmTile) * ntn;
  for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    {
      const int m0 = (tile / ntn) * kGemmTile, n0 = (tile % ntn) * tn;
      float ra[kGPerA], rb[kGPerB];
      bool bk = bkmaj(0);
      auto fetch = [&](int k0, bool kmaj) {   // raw values, clamped addresses
#pragma unroll
        for (int q = 0; q < kGPerA; ++q) {
          int mm, ka;
          a_at(q, mm, ka);
          ra[q] = fa(min(m0 + mm, M - 1), min(k0 + ka, K - 1));
        }
#pragma unroll
        for (int q = 0; q < nb; ++q) {
          int kb, nn;
          b_at(kmaj, q, kb, nn);
          rb[q] = fb(min(k0 + kb, K - 1), min(n0 + nn, N - 1));
        }
      };
      fetch(0, bk);
      f32x16 acc0 = {}, acc1 = {};
      for (int k0 = 0; k0 < K; k0 += kGk) {
#pragma unroll
        for (int q = 0; q < kGPerA; ++q) {
          int mm, ka;
          a_at(q, mm, ka);
          As[ka * (kGemmTile + 1) + mm] = (m0 + mm < M && k0 + ka < K) ? ra[q] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < nb; ++q) {
          int kb, nn;
          b_at(bk, q, kb, nn);
          Bs[kb * (kGN + 1) + nn] = (n0 + nn < N && k0 + kb < K) ? rb[q] : 0.f;
        }
        __syncthreads();
        // the next slice's loads are in flight during the products below (past
        // the last slice they reread the clamped last column: unused)
        bk = bkmaj(k0 + kGk);
        fetch(k0 + kGk, bk);
        constexpr int ksteps = kGk / ksplit;   // k rows of the slice this wave multiplies
#pragma unroll
        for (int kk = 0; kk < ksteps; kk += 4) {
          const int k = kh * ksteps + kk + lk;
          const float* ar = As + k * (kGemmTile + 1) + wm + li;
          const float* br = Bs + k * (kGN + 1) + wn + li;
          acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[0], br[0], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[2 * (kGemmTile + 1)], br[2 * (kGN + 1)], acc1, 0, 0, 0);
        }
        __syncthreads();
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc0[r] += acc1[r];
      if constexpr (ksplit > 1) {
        // the block's other waves hand their partial sums to its first wave
        // through the (now free) staging area
        if (kh) {
          float* red = As + ((blk * (ksplit - 1) + kh - 1) * 64 + lane) * 17;
#pragma unroll
          for (int r = 0; r < 16; ++r) red[r] = acc0[r];
        }
        __syncthreads();
        if (!kh) {
#pragma unroll
          for (int h = 0; h < ksplit - 1; ++h) {
            const float* red = As + ((blk * (ksplit - 1) + h) * 64 + lane) * 17;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc0[r] += red[r];
          }
        }
        __syncthreads();
      }
      if (!kh) {
        // epilogue in groups of kEpiGroup accumulator rows: every pre() read
        // of a group is issued before its epi() stores (a store may alias a
        // later element's read, so reads are never moved past it)
#pragma unroll
        for (int g = 0; g < 16; g += kEpiGroup) {
          PreT pv[kEpiGroup];
#pragma unroll
          for (int r = g; r < g + kEpiGroup; ++r) {
            const int mc = min(m0 + wm + 8 * (r >> 2) + 4 * lk + (r & 3), M - 1), n = n0 + wn + li;
            pv[r - g] = pre(mc, min(n, N - 1));
          }
#pragma unroll
          for (int r = g; r < g + kEpiGroup; ++r) {
            const int m = m0 + wm + 8 * (r >> 2) + 4 * lk + (r & 3), n = n0 + wn + li;
            epi(min(m, M - 1), min(n, N - 1), acc0[r], pv[r - g], m < M && n < N);
          }
        }
      }
    }
  }
  __syncthreads();
}

template <bool A_KMAJOR, class FA, class FB, class FBK, class FP, class FE>
__device__ void block_gemm(int M, int N, int K, FA fa, FB fb, FBK bkmaj, FP pre, FE epi) {
  if (N > kGemmTile)
    block_gemm_tiles<A_KMAJOR, true>(M, N, K, fa, fb, bkmaj, pre, epi);
  else
    block_gemm_tiles<A_KMAJOR, false>(M, N, K, fa, fb, bkmaj, pre, epi);
}

// the same with an epilogue that only stores: epi(m, n, value, ok)
template <bool A_KMAJOR, class FA, class FB, class FBK, class FE>
__device__ void block_gemm(int M, int N, int K, FA fa, FB fb, FBK bkmaj, FE epi) {
  block_gemm<A_KMAJOR>(
      M, N, K, fa, fb, bkmaj, [](int, int) { return 0.f; },
      [=](int m, int n, float x, float, bool ok) { epi(m, n, x, ok); });
}

// the B slice's layout when it is the same for every slice
constexpr auto kB_KMAJOR = [](int) { return true; };
constexpr auto kB_NMAJOR = [](int) { return false; };

// Loops over global arrays issue their reads in batches ahead of their
// stores: a store may alias any later read, so a loop that stores every
// iteration would otherwise wait out a full memory round trip per iteration.
constexpr int kBatch = 8;

// Elementwise pass of the workgroup over [0, count): value = load(e) for
// kBatch iterations per thread, then store(e, value) for each.  No barrier
// inside.
template <class FL, class FS>
__device__ void each(int count, FL load, FS store) {
  using T = decltype(load(0));
  for (int e0 = threadIdx.x; e0 < count; e0 += kGemmThreads * kBatch) {
    T v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = load(min(e0 + j * kGemmThreads, count - 1));
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (e0 + j * kGemmThreads < count) store(e0 + j * kGemmThreads, v[j]);
  }
}

}  // namespace
}  // namespace titans
