// Transposed matrix-core operands read straight from row-major LDS tiles, for the staged
// and backward kernels: the transposing LDS read of gfx950 for 16-bit data, strided reads
// for fp32.
#pragma once

#include "gdn_device.h"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16): within each group of 16 lanes,
// if lane c of group g addresses row R0 + 4 g + c / 4, columns C0 + 4 (c % 4) .. + 3 of a
// row-major matrix M, lane c receives M[R0 + 4 g + e][C0 + c], e = 0..3.
__device__ __forceinline__ bf16x4 read_tr4(const bf16* p) {
  const s16x4 r =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// The k-contiguous operand fragment of M^T (rows n0 + l%16, k = k0 + 8 (l/16) + 0..7; the
// layout of frag_ld) from row-major M [k][n] in LDS: two transposing reads in bf16, a
// strided read in fp32.
template <typename TI>
__device__ __forceinline__ typename Mma<TI>::frag frag_tr(const TI* M, int ld, int n0, int k0) {
  const int l = lane_id(), c = l & 15, g = l >> 4;
  if constexpr (sizeof(TI) == 2) {
    const TI* p = M + (k0 + 8 * g + (c >> 2)) * ld + n0 + 4 * (c & 3);
    const bf16x4 a = read_tr4(p), b = read_tr4(p + 4 * ld);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return M[(k0 + g) * ld + n0 + c];
  }
}

// A block of matrix-core products sharing fragment reads: per k-step over [0, K), the NA
// A fragments fa(i, k) and NB B fragments fb(j, k) are read once, then fm(a, b) issues the
// products (each fragment serves several tiles: fewer LDS reads per product).
template <typename E, int K, int NA, int NB, typename FA, typename FB, typename FM>
__device__ __forceinline__ void mma_steps(FA fa, FB fb, FM fm) {
#pragma unroll
  for (int k = 0; k < K; k += Mma<E>::KS) {
    typename Mma<E>::frag a[NA], b[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i) a[i] = fa(i, k);
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = fb(j, k);
    fm(a, b);
  }
}

}  // namespace gdn
