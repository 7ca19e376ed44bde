// Workgroup-wide fp32 contraction on the matrix cores, shared by the
// shape-generic forward sweep and the chunk-wise backward sweep (device code
// only; each translation unit gets its own copy).
#pragma once

#include <hip/hip_runtime.h>

namespace titans {
namespace {

constexpr int kGemmThreads = 256;   // workgroup size every caller launches with
constexpr int kGemmTile = 64;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C[M x N] = sum_k A(m, k) B(k, n), handed to epi(m, n, value).  The whole
// workgroup cooperates; operands come through accessors (global/L2 reads)
// and are staged through LDS in kGk-deep slices, the next slice's operands
// loaded into registers while the current one is multiplied.  Output tiles
// are 64 x 128 when N > 64 (each of the four waves computes a 32 x 64 part
// as two 32 x 32 blocks), else 64 x 64 (each wave a 32 x 32 quarter with
// the slice's even and odd k-pairs in two accumulators, summed at the end),
// so every wave keeps two independent chains of the fp32 matrix instruction
// v_mfma_f32_32x32x2_f32 (lane l supplies A[l%32][l/32] and B[l/32][l%32];
// accumulator register r holds row 8(r/4) + 4(l/32) + r%4, column l%32) and
// the arithmetic stays fp32.  The accessors are read in the order that keeps
// a wavefront's loads on few cache lines: A_KMAJOR says A(m, k) is
// contiguous in k (else in m); bkmaj(k0) says whether the B slice starting
// at k0 is contiguous in k (else in n).
//
// So that a wave keeps all of a slice's loads in flight at once, the
// accessors and the epilogue are called unconditionally, with indices
// clamped into range (M, N, K >= 1): fa(m, k) and fb(k, n) must be
// branch-free reads of valid addresses; operands outside the product are
// zeroed when staged.  The epilogue is split in two: pre(m, n) reads what
// the element's update needs (any value type), epi(m, n, value, pre, ok)
// stores, only where ok is set.
constexpr int kGk = 32;                                  // k per staged slice
constexpr int kGN = 2 * kGemmTile;                       // output columns per wide tile
constexpr int kGPerA = kGemmTile * kGk / kGemmThreads;   // A elements per thread per slice
constexpr int kGPerB = kGN * kGk / kGemmThreads;         // B elements per thread per wide slice
constexpr int kEpiGroup = 8;                             // accumulator rows per epilogue group
constexpr int kGemmLdsFloats = kGk * (kGemmTile + 1) + kGk * (kGN + 1);

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
  const int lane = tid & 63, wv = tid >> 6;
  constexpr bool wide = WIDE;
  constexpr int tn = wide ? kGN : kGemmTile;       // output columns per tile
  constexpr int nb = wide ? kGPerB : kGPerB / 2;   // B elements per thread per slice
  const int wm = (wv >> 1) * 32, wn = (wv & 1) * (wide ? 64 : 32);
  const int li = lane & 31, lk = lane >> 5;
  auto a_at = [&](int q, int& mm, int& ka) {
    const int e = tid + q * kGemmThreads;
    if (A_KMAJOR) { mm = e / kGk; ka = e % kGk; } else { ka = e / kGemmTile; mm = e % kGemmTile; }
  };
  auto b_at = [&](bool kmaj, int q, int& kb, int& nn) {
    const int e = tid + q * kGemmThreads;
    if (kmaj) { nn = e / kGk; kb = e % kGk; } else { kb = e / tn; nn = e % tn; }
  };
  for (int m0 = 0; m0 < M; m0 += kGemmTile) {
    for (int n0 = 0; n0 < N; n0 += tn) {
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
        if constexpr (wide) {
#pragma unroll
          for (int kk = 0; kk < kGk; kk += 2) {
            const float a = As[(kk + lk) * (kGemmTile + 1) + wm + li];
            const float* br = Bs + (kk + lk) * (kGN + 1) + wn + li;
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, br[0], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, br[32], acc1, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < kGk; kk += 4) {
            const float* ar = As + (kk + lk) * (kGemmTile + 1) + wm + li;
            const float* br = Bs + (kk + lk) * (kGN + 1) + wn + li;
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[0], br[0], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[2 * (kGemmTile + 1)], br[2 * (kGN + 1)], acc1, 0, 0, 0);
          }
        }
        __syncthreads();
      }
      // epilogue in groups of kEpiGroup accumulator rows: every pre() read
      // of a group is issued before its epi() stores (a store may alias a
      // later element's read, so reads are never moved past it)
#pragma unroll
      for (int g = 0; g < 16; g += kEpiGroup) {
        PreT pv0[kEpiGroup], pv1[kEpiGroup];
#pragma unroll
        for (int r = g; r < g + kEpiGroup; ++r) {
          const int mc = min(m0 + wm + 8 * (r >> 2) + 4 * lk + (r & 3), M - 1), n = n0 + wn + li;
          pv0[r - g] = pre(mc, min(n, N - 1));
          if constexpr (wide) pv1[r - g] = pre(mc, min(n + 32, N - 1));
        }
#pragma unroll
        for (int r = g; r < g + kEpiGroup; ++r) {
          const int m = m0 + wm + 8 * (r >> 2) + 4 * lk + (r & 3), n = n0 + wn + li;
          const int mc = min(m, M - 1);
          if constexpr (wide) {
            epi(mc, min(n, N - 1), acc0[r], pv0[r - g], m < M && n < N);
            epi(mc, min(n + 32, N - 1), acc1[r], pv1[r - g], m < M && n + 32 < N);
          } else {
            epi(mc, min(n, N - 1), acc0[r] + acc1[r], pv0[r - g], m < M && n < N);
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
