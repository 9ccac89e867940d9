// Blocked inverse of the unit lower-triangular chunk matrix (I + A), A strictly lower:
// the solve_tril stage of the MegaGDN-PTO page (section 4.4), which inverts the
// lower-triangular chunk matrix recursively by sub-blocks on the matrix unit.
//
// gfx950 design: the 16 x 16 diagonal blocks are inverted in fp32 by forward
// substitution, one column per lane (VALU); then blocks are merged pairwise
// (16 -> 32 -> 64 -> C) with   T21 = -T22 (A21 T11)   on the matrix cores, one wave per
// 16-column slice of T21.  A21 T11 stays in that wave's registers and is fed straight
// back as the B operand of the second product (see gdn_device.h), so a level needs one
// barrier.
//
// Storage (LDS):
//   sA  [C][ldA] TS   A's off-diagonal 16 x 16 blocks, row-major (diagonal blocks unused)
//   sAd [C/16][16][17] f32   A's diagonal blocks
//   sM  [C][ldM] TS   result: M[i][j] = T[max(i,j)][min(i,j)], i.e. T = (I + A)^-1 below
//                     and on the diagonal, T^T above it (both operand orientations in one
//                     buffer; readers mask the half they do not want).  sM may be sA itself
//                     (in place): A's diagonal blocks are not read from sA, and each
//                     off-diagonal block of A is read in the level that overwrites it.
#pragma once

#include "gdn_device.h"

namespace gdn {

constexpr int kAdLd = 17;  // leading dim of a diagonal block in sAd

template <int NW, int C, typename TS>
__device__ __forceinline__ void solve_diag_column(const float* sAd, TS* sM, int ldM, int t);

// Inverse of each 16 x 16 diagonal block, one column per thread t < C.
template <int NW, int C, typename TS>
__device__ __forceinline__ void solve_diag_blocks(const float* sAd, TS* sM, int ldM, int t) {
  if (t < C) solve_diag_column<NW, C, TS>(sAd, sM, ldM, t);
}

template <int NW, int C, typename TS>
__device__ __forceinline__ void solve_diag_column(const float* sAd, TS* sM, int ldM, int t) {
  {
    const int b = t >> 4, c = t & 15;
    const float* Ab = sAd + b * 16 * kAdLd;
    // Forward substitution down column c, column-oriented: once x_m is final, every later
    // row's sum takes its term -A[i][m] x_m at once (independent FMAs), so the dependent
    // chain is one FMA per row rather than one per term.  Each row still sums its terms in
    // the order m = 0, 1, ... from the identity's entry, as row-by-row substitution does.
    // Columns of A are loaded two ahead.
    float x[16];
    float ca[16], cb[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = (i == c) ? 1.f : 0.f;
      ca[i] = i > 0 ? Ab[i * kAdLd + 0] : 0.f;
      cb[i] = i > 1 ? Ab[i * kAdLd + 1] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < 15; ++m) {
      const float xm = x[m];
#pragma unroll
      for (int i = m + 1; i < 16; ++i) x[i] = fmaf(-ca[i], xm, x[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ca[i] = cb[i];
        cb[i] = (m + 2 < 16 && i > m + 2) ? Ab[i * kAdLd + m + 2] : 0.f;
      }
    }
    const int base = 16 * b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i >= c) {
        sM[(base + i) * ldM + base + c] = (TS)x[i];
        sM[(base + c) * ldM + base + i] = (TS)x[i];
      }
    }
  }
}

// One merge level: pairs of S x S inverse blocks become 2S x 2S blocks.  InPlace: sA and
// sM are the same storage (A's off-diagonal blocks are overwritten by T's), so every
// wave first reads its A21 blocks, then a barrier, then T21 is written.
template <int NW, int C, typename TS, int S, bool InPlace>
__device__ __forceinline__ void solve_level(const TS* sA, int ldA, TS* sM, int ldM, int w,
                                            int l) {
  constexpr int NB = S / 16;                 // 16-blocks per half of a merged pair
  constexpr int NJOBS = (C / (2 * S)) * NB;  // (pair, 16-column slice) jobs = C / 32
  constexpr int JPW = (NJOBS + NW - 1) / NW;
  constexpr int KS = Mma<TS>::KS;
  constexpr int KPL = Mma<TS>::KPL;
  typedef typename Mma<TS>::frag frag;
  f32x4 y[JPW][NB];
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int job = w + jj * NW;
    if (job < NJOBS) {
      const int p = job / NB, J = job % NB;
      const int o = 2 * S * p;
      // Y[:, J] = A21 T11[:, J]; T11 is lower, so k starts at the slice's first column.
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) y[jj][kb] = zero4();
      const int ncol = o + 16 * J + (l & 15);
      for (int k = o + 16 * J; k < o + S; k += KS) {
        const int kl = k + KPL * (l >> 4);
        frag b = frag_ld<TS>(sM, ldM, o + 16 * J, k, l);  // row ncol of M: T^T above diagonal
        if constexpr (KPL == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kl + e < ncol || kl + e >= o + S) b[e] = (TS)0.f;
        } else {
          if (kl < ncol || kl >= o + S) b = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          frag a = frag_ld<TS>(sA, ldA, o + S + 16 * kb, k, l);
          if constexpr (KPL == 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (kl + e >= o + S) a[e] = (TS)0.f;
          } else {
            if (kl >= o + S) a = 0.f;
          }
          y[jj][kb] = Mma<TS>::mma(a, b, y[jj][kb]);
        }
      }
    }
  }
  if constexpr (InPlace && NW > 1) __syncthreads();
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int job = w + jj * NW;
    if (job < NJOBS) {
      const int p = job / NB, J = job % NB;
      const int o = 2 * S * p;
      // T21[I, J] = -sum_{kb <= I} T22[I, kb] Y[kb, J]; T22 is read from M's lower half.
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        f32x4 acc = zero4();
        mma_accB<TS, NB, true>(acc, sM, ldM, o + S + 16 * I, o + S, y[jj], I + 1, 0, l);
        const int R0 = o + S + 16 * I + 4 * (l >> 4);
        const int Cc = o + 16 * J + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const TS val = (TS)(-acc[e]);
          sM[(R0 + e) * ldM + Cc] = val;
          sM[Cc * ldM + R0 + e] = val;
        }
      }
    }
  }
  if constexpr (NW > 1) __syncthreads();
}

// Full solve.  Precondition: sA / sAd written and visible (barrier done).  Ends with a
// barrier, after which sM holds the result.  tid / w / l: thread, wave and lane index
// (passed in so callers can keep them opaque).  InPlace: sM == sA.
template <int NW, int C, typename TS, bool InPlace = false>
__device__ __forceinline__ void solve_tril(const TS* sA, int ldA, const float* sAd, TS* sM,
                                           int ldM, int tid = threadIdx.x, int w = wave_id(),
                                           int l = lane_id()) {
  static_assert(C == 64 || C == 128, "chunk size");
  static_assert(NW * kWave >= C, "one lane per diagonal-block column");
  solve_diag_blocks<NW, C, TS>(sAd, sM, ldM, tid);
  __syncthreads();
  solve_level<NW, C, TS, 16, InPlace>(sA, ldA, sM, ldM, w, l);
  solve_level<NW, C, TS, 32, InPlace>(sA, ldA, sM, ldM, w, l);
  if constexpr (C == 128) solve_level<NW, C, TS, 64, InPlace>(sA, ldA, sM, ldM, w, l);
}

}  // namespace gdn
