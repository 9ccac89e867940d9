// Device-side building blocks shared by the staged and fused kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used everywhere (v_mfma_f32_16x16x32_{bf16,f16} and
// v_mfma_f32_16x16x4_f32, wave64):
//   * an output tile is 16 x 16 fp32; lane l holds rows 4*(l/16) + i (i = 0..3) of column
//     l % 16 ("accumulator layout");
//   * the A operand of a 16 x 16 tile reads, in lane l, row l % 16 and KPL consecutive k
//     values starting at k0 + KPL*(l/16); the B operand reads column l % 16 the same way.
//     Operands staged in LDS are therefore stored "k-contiguous": A as [row][k], B as
//     [col][k] (B transposed);
//   * since A and B only need to agree on which k each (lane, element) slot carries, an
//     accumulator tile can be fed back as a B operand whose k runs over the tile's rows:
//     slot (lane, i < 4) carries k = 16*kb + 4*(l/16) + i of block kb and slot i + 4 the
//     same row of block kb + 1.  The A operand then reads its two 4-element groups from
//     LDS at those k.  This keeps state, residuals and new values in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

template <typename E> __device__ __forceinline__ float to_f32(E x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f32(float x) { return (E)x; }

// Operand traits for the three matrix-core shapes in use.
template <typename E> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KPL = 8;   // k values one lane supplies
  static constexpr int KS = 32;   // k per instruction
  typedef bf16x8 frag;
  typedef bf16x4 half;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<f16> {
  static constexpr int KPL = 8;
  static constexpr int KS = 32;
  typedef f16x8 frag;
  typedef f16x4 half;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KPL = 1;
  static constexpr int KS = 4;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row padding (elements) for k-contiguous LDS operands: 16 bytes, so that the 16 rows
// a fragment load touches fall in different bank groups.
template <typename E> constexpr int pad_of() { return 16 / (int)sizeof(E); }

// Standard fragment load from a k-contiguous LDS matrix m[row][k] (leading dim ld).
template <typename E>
__device__ __forceinline__ typename Mma<E>::frag frag_ld(const E* m, int ld, int row0, int k0,
                                                         int l = lane_id()) {
  const E* p = m + (row0 + (l & 15)) * ld + k0 + Mma<E>::KPL * (l >> 4);
  if constexpr (Mma<E>::KPL == 8) {
    return *reinterpret_cast<const typename Mma<E>::frag*>(p);
  } else {
    return *p;
  }
}

// acc += A[row0.., k] * B[col0.., k] over k in [k0, k1) (k1 - k0 a multiple of KS), both
// operands k-contiguous in LDS.
template <typename E>
__device__ __forceinline__ void mma_lds(f32x4& acc, const E* A, int lda, int arow0,
                                        const E* B, int ldb, int bcol0, int k0, int k1,
                                        int l = lane_id()) {
  for (int k = k0; k < k1; k += Mma<E>::KS)
    acc = Mma<E>::mma(frag_ld<E>(A, lda, arow0, k, l), frag_ld<E>(B, ldb, bcol0, k, l), acc);
}

// ---------------------------------------------------------------------------------------
// Contraction with the B operand taken from accumulator tiles (see the header comment).
//   acc += sum over kb < nkb of  A[arow0 + r][16*kb + c] * Bt[kb][c][col]
// where Bt[kb] is an accumulator tile whose rows run over k.  A is k-contiguous in LDS
// (row-major [row][k], leading dim lda, k offset koff).  If `mask_upper` the A element is
// taken as zero where its k exceeds its row index (row and k both offset by `diag`):
// used to read a lower-triangular matrix out of a storage that holds other data above
// the diagonal.
template <typename E, int NKB, bool MaskUpper = false>
__device__ __forceinline__ void mma_accB(f32x4& acc, const E* A, int lda, int arow0, int koff,
                                         const f32x4* Bt, int nkb, int diag = 0,
                                         int l = lane_id()) {
  const int r = arow0 + (l & 15);
  const int g4 = 4 * (l >> 4);
  if constexpr (Mma<E>::KPL == 8) {
    typedef typename Mma<E>::frag frag;
    typedef typename Mma<E>::half half;
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2) {
      if (kb < nkb) {
        const bool two = (kb + 1 < NKB) && (kb + 1 < nkb);
        const E* p0 = A + r * lda + koff + 16 * kb + g4;
        half x0 = *reinterpret_cast<const half*>(p0);
        half x1 = two ? *reinterpret_cast<const half*>(p0 + 16) : half{0, 0, 0, 0};
        if constexpr (MaskUpper) {
          const int row = r - diag;
          const int k0 = 16 * kb + g4 + koff - diag;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (k0 + i > row) x0[i] = (E)0.f;
            if (k0 + 16 + i > row) x1[i] = (E)0.f;
          }
        }
        const half b0 = __builtin_convertvector(Bt[kb], half);
        const half b1 = two ? __builtin_convertvector(Bt[kb + 1], half) : half{0, 0, 0, 0};
        const frag a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        const frag b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = Mma<E>::mma(a, b, acc);
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb < nkb) {
        const E* p0 = A + r * lda + koff + 16 * kb + g4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          E x = p0[i];
          if constexpr (MaskUpper) {
            if (16 * kb + g4 + i + koff - diag > r - diag) x = (E)0.f;
          }
          acc = Mma<E>::mma(x, Bt[kb][i], acc);
        }
      }
    }
  }
}

// B tiles may be held as fp32 accumulators (converted at use) or already as 16-bit
// 4-vectors (the form they take as operands).
template <typename H> __device__ __forceinline__ H as_half(const f32x4& x) {
  return __builtin_convertvector(x, H);
}
template <typename H> __device__ __forceinline__ H as_half(const H& x) { return x; }

// Same contraction for NJ outputs that share the A operand; one A fragment load feeds NJ
// matrix-core instructions.
//   acc[j * AJ] += A * B_j,  B_j block kb = Bt[j * BJ + kb * BK].
template <typename E, int NKB, int NJ, bool MaskUpper = false, int AJ = 1, int BJ = NKB,
          int BK = 1, typename BT = f32x4>
__device__ __forceinline__ void mma_accB_n(f32x4* acc, const E* A, int lda, int arow0, int koff,
                                           const BT* Bt, int nkb, int diag = 0,
                                           int l = lane_id()) {
  const int r = arow0 + (l & 15);
  const int g4 = 4 * (l >> 4);
  static_assert(Mma<E>::KPL == 8, "16-bit operands");
  typedef typename Mma<E>::frag frag;
  typedef typename Mma<E>::half half;
#pragma unroll
  for (int kb = 0; kb < NKB; kb += 2) {
    if (kb < nkb) {
      const bool two = (kb + 1 < NKB) && (kb + 1 < nkb);
      const E* p0 = A + r * lda + koff + 16 * kb + g4;
      half x0 = *reinterpret_cast<const half*>(p0);
      half x1 = two ? *reinterpret_cast<const half*>(p0 + 16) : half{0, 0, 0, 0};
      if constexpr (MaskUpper) {
        const int row = r - diag;
        const int k0 = 16 * kb + g4 + koff - diag;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (k0 + i > row) x0[i] = (E)0.f;
          if (k0 + 16 + i > row) x1[i] = (E)0.f;
        }
      }
      const frag a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const half b0 = as_half<half>(Bt[j * BJ + kb * BK]);
        const half b1 = two ? as_half<half>(Bt[j * BJ + (kb + 1) * BK]) : half{0, 0, 0, 0};
        acc[j * AJ] = Mma<E>::mma(a, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                  acc[j * AJ]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Software-pipelined form of the accumulator-fed contraction, for a run of NR output row
// blocks that share the B tiles: the A fragments of row block r + 1 are loaded from LDS
// before the matrix-core work of row block r is issued, so a single wave per SIMD keeps
// its LDS latency hidden.
template <typename E, int NPAIR>
struct ARow {
  typename Mma<E>::frag f[NPAIR];
};

// A fragments of one 16-row block: pair p covers k blocks 2p and 2p + 1 (only the first
// `nkb` k blocks are real; the rest read as zero).
template <typename E, int NPAIR>
__device__ __forceinline__ void load_arow(ARow<E, NPAIR>& a, const E* A, int lda, int row0,
                                          int koff, int nkb, int l) {
  typedef typename Mma<E>::half half;
  const E* p0 = A + (row0 + (l & 15)) * lda + koff + 4 * (l >> 4);
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    half x0 = half{0, 0, 0, 0}, x1 = half{0, 0, 0, 0};
    if (2 * p < nkb) x0 = *reinterpret_cast<const half*>(p0 + 32 * p);
    if (2 * p + 1 < nkb) x1 = *reinterpret_cast<const half*>(p0 + 32 * p + 16);
    a.f[p] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

//   acc[j * AJ] += A_row * B_j,  B_j block kb = Bt[j * BJ + kb * BK] (16-bit 4-vectors).
template <typename E, int NPAIR, int NJ, int AJ, int BJ, int BK>
__device__ __forceinline__ void mma_arow(f32x4* acc, const ARow<E, NPAIR>& a,
                                         const typename Mma<E>::half* Bt, int nkb) {
  typedef typename Mma<E>::half half;
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    if (2 * p < nkb) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const half b0 = Bt[j * BJ + 2 * p * BK];
        const half b1 = (2 * p + 1 < nkb) ? Bt[j * BJ + (2 * p + 1) * BK] : half{0, 0, 0, 0};
        acc[j * AJ] = Mma<E>::mma(a.f[p], __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6,
                                                                  7), acc[j * AJ]);
      }
    }
  }
}

// Keep the scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Make the compiler treat a value as changed here, so address arithmetic derived from it is
// not hoisted out of a loop (and kept live across it).
template <typename T> __device__ __forceinline__ void opaque(T& x) { asm volatile("" : "+v"(x)); }

// x from another lane by a DPP pattern (CTRL), in the rows (ROWS) and banks (BANKS) it
// enables; lanes it leaves out, and lanes whose source lies outside the pattern, get 0.
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, ROWS, BANKS, true));
}

// Inclusive prefix sum across a wave, in the VALU by DPP (no LDS traffic): a Hillis-Steele
// scan within each 16-lane row (shifts by 1, 2, 4, 8 lanes), then the row totals carried
// down: the last lane of rows 0 and 2 into rows 1 and 3, and lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_f<0x111>(x);        // row_shr 1
  x += dpp_f<0x112>(x);        // row_shr 2
  x += dpp_f<0x114>(x);        // row_shr 4
  x += dpp_f<0x118>(x);        // row_shr 8
  x += dpp_f<0x142, 0xA>(x);   // row_bcast 15, rows 1 and 3
  x += dpp_f<0x143, 0xC>(x);   // row_bcast 31, rows 2 and 3
  return x;
}

__device__ __forceinline__ int wave_incl_scan_int(int x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (l >= d) x += y;
  }
  return x;
}

// beta is bf16 or fp32 (runtime flag): read element i as fp32.
// One workgroup's copy of a ROWS x COLS block of TI (row r at src + r * stride; rows
// r >= len read as zero, len >= 1) in RB x V sub-blocks, V = 16 / sizeof(TI) and RB chosen
// so that every thread holds one: RB rows of one 16-byte vector each.  Eight lanes cover
// 128 contiguous bytes of a source row.  The loads are unconditional (rows past len read
// the last valid row) and nothing touches their results until a store zeroes the rows past
// len, so a load issued phases ahead stays in flight until its data is stored.  Stored
// natural (dst[r * ld + c], 16-byte LDS stores) or transposed in registers (dst[c * ld + r],
// RB-element stores).  tile_copy_fits tells whether a shape gives every thread exactly one
// sub-block.
template <typename TI, int ROWS, int COLS, int NTH>
constexpr bool tile_copy_fits() {
  constexpr int V = 16 / (int)sizeof(TI), BC = COLS / V;
  constexpr int RB = ROWS * BC / NTH < V ? ROWS * BC / NTH : V;
  return RB >= 1 && ROWS % RB == 0 && (ROWS / RB) % 8 == 0 && BC % 8 == 0 &&
         (ROWS / RB) * BC == NTH;
}

template <typename TI, int ROWS, int COLS, int NTH>
struct TileCopy {
  static constexpr int V = 16 / (int)sizeof(TI), BC = COLS / V;
  static constexpr int RB = ROWS * BC / NTH < V ? ROWS * BC / NTH : V;
  static constexpr int BR = RB > 0 ? ROWS / RB : 0, NB = BR * BC;
  static_assert(tile_copy_fits<TI, ROWS, COLS, NTH>(), "block shape");
  union Vec {
    uint4 u;
    TI e[V];
  };
  typedef TI Col __attribute__((ext_vector_type(RB > 1 ? RB : 2)));
  Vec in[RB];
  int r0, c0, len;

  __device__ __forceinline__ void load(const TI* src, long stride, int len_) {
    const int lo = threadIdx.x & 63, hi = threadIdx.x >> 6;
    const int bc = (lo & 7) + 8 * (hi % (BC / 8)), br = (lo >> 3) + 8 * (hi / (BC / 8));
    r0 = RB * br;
    c0 = V * bc;
    len = len_;
#pragma unroll
    for (int a = 0; a < RB; ++a)
      in[a].u = *reinterpret_cast<const uint4*>(src + (long)min(r0 + a, len - 1) * stride + c0);
  }
  __device__ __forceinline__ Vec row(int a) const {
    Vec x;
    x.u = r0 + a < len ? in[a].u : make_uint4(0, 0, 0, 0);
    return x;
  }
  __device__ __forceinline__ void store_nat(TI* dst, int ld) const {
#pragma unroll
    for (int a = 0; a < RB; ++a) *reinterpret_cast<uint4*>(dst + (r0 + a) * ld + c0) = row(a).u;
  }
  __device__ __forceinline__ void store_trn(TI* dst, int ld) const {
    Vec x[RB];
#pragma unroll
    for (int a = 0; a < RB; ++a) x[a] = row(a);
#pragma unroll
    for (int b = 0; b < V; ++b) {
      if constexpr (RB == 1) {
        dst[(c0 + b) * ld + r0] = x[0].e[b];
      } else {
        Col o;
#pragma unroll
        for (int a = 0; a < RB; ++a) o[a] = x[a].e[b];
        *reinterpret_cast<Col*>(dst + (c0 + b) * ld + r0) = o;
      }
    }
  }
  // sum over the held elements of x * other[r][c] (other natural, leading dimension ld)
  __device__ __forceinline__ float dot_nat(const TI* other, int ld) const {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < RB; ++a) {
      const Vec x = row(a);
      Vec o;
      o.u = *reinterpret_cast<const uint4*>(other + (r0 + a) * ld + c0);
#pragma unroll
      for (int b = 0; b < V; ++b) s += (float)x.e[b] * (float)o.e[b];
    }
    return s;
  }
};

__device__ __forceinline__ float load_beta(const void* beta, int f32, long i) {
  return f32 ? static_cast<const float*>(beta)[i] : (float)static_cast<const bf16*>(beta)[i];
}

// Sequence span [start, start + len) of sequence n, clamped to [0, Ttot].
__device__ __forceinline__ void seq_span(const int32_t* cu, int n, int T, int Ttot, int& start,
                                         int& len) {
  int s, e;
  if (cu) {
    s = cu[n];
    e = cu[n + 1];
  } else {
    s = n * T;
    e = s + T;
  }
  s = min(max(s, 0), Ttot);
  e = min(max(e, s), Ttot);
  start = s;
  len = e - s;
}

}  // namespace gdn
