// Fused single-launch chunked Gated DeltaNet forward (the megakernel idea of the
// MegaGDN-PTO page, sections 1.3 and 4.5: all seven stages in one launch, intermediates
// kept on chip), designed for gfx950.
//
// One workgroup owns one (sequence, value head) and walks its chunks in order; nothing
// crosses workgroups, so no grid barrier is needed (the page's all-core SyncAll barrier
// has no counterpart here).  D/32 waves, one per SIMD with a 512-register budget; wave w
// owns 32 state columns as two 16-wide matrix-core column blocks, for all Dk rows, kept as
// fp32 accumulator tiles, so the recurrent chain K h -> R -> T R -> (o, h) never leaves
// registers and every A-operand fragment feeds two matrix-core instructions.  Column c of
// block j of wave w is state column dv = 32 w + 2 c + j, so each lane's two columns are
// adjacent in memory (4-byte V / o and 8-byte h0 / ht accesses).  Per chunk, with G the
// in-chunk prefix sum of g:
//
//   A    = (K K^T) * beta_i e^{G_i-G_j}, i > j            (scaled_dot_kkt, section 4.2)
//   T    = (I + A)^-1                                      (solve_tril, section 4.4)
//   R    = diag(beta) (V - diag(e^G) K h)                  (wy_fast + chunk_h, 4.3):
//   v_new = T R  = U - W h                                  T applied once to V - e^G K h
//   o    = scale (diag(e^G) Q h + (Q K^T * e^{G_i-G_j})_{i>=j} v_new)       (chunk_o)
//   h    = e^{G_last} h + K^T (e^{G_last-G} v_new)          (chunk_h, TileLang page step 1)
//
// Applying T to (V - e^G K h) instead of forming W = T diag(beta e^G) K and U = T diag(beta)
// V separately is exact algebra (v_new = U - W h) and saves the C x C x Dk product W.
//
// LDS: four slabs re-used by phase —
//   S0: K            -> A (fp16, off-diagonal blocks) -> T (solved in place; bf16, lower)
//   S1: Q                                (read again for Q h in the output phase)
//   S2: V            -> P = gated, masked Q K^T (bf16)
//   S3: K^T scaled by e^{G_last - G}
// plus the fp32 diagonal blocks of A and the chunk's gate vectors (G, e^G, beta,
// e^{G_last-G}), which wave 0 computes for the next chunk at the end of the current one
// (double-buffered).  The next chunk's K, Q and V are copied from HBM straight into their
// slabs (global_load_lds, no register staging) as soon as the current chunk is done with
// each slab: K after T R, Q and V after the output.  K, Q, V rows are unpadded with the
// 16-byte chunk index XOR-swizzled by the row, which keeps fragment reads conflict-free
// and matches the lane order of the direct-to-LDS copy.  R and v_new live in registers in
// the bf16 form in which they feed the matrix cores.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_solve.h"

namespace gdn {

namespace {

// 16-column state blocks per wave: 2 -> D/32 waves, one per SIMD with up to 512
// registers (spill-free; every A fragment feeds two matrix-core instructions); 1 -> D/16
// waves, two per SIMD with 256 registers each.
#ifndef GDN_FUSED_NJ
#define GDN_FUSED_NJ 2
#endif
constexpr int kFusedNJ = GDN_FUSED_NJ;


template <int D, int C, int NJ_>
struct FusedCfg {
  static constexpr int NJ = NJ_;          // 16-column blocks per wave
  static constexpr int NW = D / (16 * NJ);  // waves
  static constexpr int NTH = NW * kWave;  // = 4 D / NJ (the launch bound)
  static constexpr int NT = C / 16;       // token blocks per chunk
  static constexpr int NDK = D / 16;      // key blocks
  static constexpr int CPR = D / 8;       // 16-byte pieces per q/k/v row
  static constexpr int LDC = C + 8;       // row of a [*][C] 16-bit operand (A, T, P)
  static constexpr int LDT = C + 12;      // row of K^T (8-byte reads; spreads the writes)
  static constexpr int SLAB_TILE = C * D;                                    // swizzled rows
  static constexpr int SLAB_SQ = C * LDC;                                    // padded C x C
  static constexpr int SLAB = SLAB_TILE > SLAB_SQ ? SLAB_TILE : SLAB_SQ;    // elements
  static constexpr int KT = D * LDT;
  static constexpr int RPI = 1024 / (2 * D);        // rows per direct-to-LDS instruction
  static constexpr int NDMA = C / RPI / NW;         // such instructions per wave per tile
  static constexpr int NLOW = NT * (NT + 1) / 2;
  static constexpr int MAXT = (NT == 2 * NW) ? NT + 1 : (NLOW + NW - 1) / NW;
  static constexpr int TPL = C / kWave;             // tokens per lane in the gate scan
  static constexpr int GATES = 2 * 4 * C;           // [2][4][C] G, e^G, beta, e^{G_last-G}
  static_assert(NDMA * NW * RPI == C, "tile covered by whole copy instructions");
  static constexpr size_t lds_bytes() {
    return (size_t)(3 * SLAB + KT) * 2 + (size_t)GATES * 4 + 2 * 4 +
           (size_t)(C / 16) * 16 * kAdLd * 4 + 8;
  }
};

// Element offset of (r, k) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int swz(int r, int k) {
  constexpr int CPR = D / 8;
  return r * D + ((((k >> 3) ^ r) & (CPR - 1)) << 3) + (k & 7);
}

// Within a 16-row block (row0 % 16 == 0) the swizzle key of lane l's row is l % 16, so
// the in-row offset of a k chunk depends on the lane only: swz(row0 + l%16, k) =
// row0 * D + swz(l%16, k).
template <int D>
__device__ __forceinline__ int swz_lane(int l, int k) {
  return swz<D>(l & 15, k);
}

// Standard 16-byte fragment (rows row0 + l%16, k0 + 8 (l/16) ...) of a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 frag_swz(const bf16* m, int row0, int k0, int l) {
  return *reinterpret_cast<const bf16x8*>(m + row0 * D + swz_lane<D>(l, k0 + 8 * (l >> 4)));
}

// A-row fragments (accumulator-fed contraction form, see gdn_device.h) of a swizzled tile.
template <int D, int NPAIR>
__device__ __forceinline__ void load_arow_swz(ARow<bf16, NPAIR>& a, const bf16* m, int row0,
                                              int l) {
  const int g4 = 4 * (l >> 4);
  const bf16* mr = m + row0 * D;
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(mr + swz_lane<D>(l, 32 * p + g4));
    const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(mr + swz_lane<D>(l, 32 * p + 16 + g4));
    a.f[p] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Issue this wave's share of the direct HBM -> LDS copy of one [C][D] tile (rows of one
// head, token stride `stride`), into the swizzled layout.  Rows past `len` re-read the
// last valid row (in bounds); the caller zeroes them once the copy has landed.
template <class F, int D>
__device__ __forceinline__ void dma_tile(bf16* tile, const bf16* src, long stride, int len,
                                         int w, int l) {
  const int slot = l % F::CPR;
#pragma unroll
  for (int j = 0; j < F::NDMA; ++j) {
    const int r0 = (w * F::NDMA + j) * F::RPI;
    const int r = r0 + l / F::CPR;
    const int c = (slot ^ r) & (F::CPR - 1);
    const int rs = min(r, len - 1);
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(src + (long)rs * stride + c * 8),
        (void __attribute__((address_space(3)))*)(tile + r0 * D), 16, 0, 0);
  }
}

// Zero rows [len, C) of a swizzled tile (a partial last chunk).
template <class F, int C>
__device__ __forceinline__ void zero_tail(bf16* tile, int len, int tid) {
  for (int i = tid + len * F::CPR; i < C * F::CPR; i += F::NTH)
    *reinterpret_cast<uint4*>(tile + i * 8) = make_uint4(0, 0, 0, 0);
}

// Wave 0: g and beta of a chunk, TPL consecutive tokens per lane (zero past len).
template <int C>
__device__ __forceinline__ void load_gates(float* ga, float* be, const float* g,
                                           const void* beta, int beta_f32, int cs, int len,
                                           int h, int H, int l) {
  constexpr int TPL = C / kWave;
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    const int t = TPL * l + r;
    ga[r] = 0.f;
    be[r] = 0.f;
    if (t < len) {
      const long gi = (long)(cs + t) * H + h;
      ga[r] = g[gi];
      be[r] = load_beta(beta, beta_f32, gi);
    }
  }
}

// Wave 0: G = in-chunk prefix sum of g (chunk_cumsum), then e^G, beta and
// e^{G_last - G} (zero past len) into sm[4][C], e^{G_last} into *misc.
template <int C>
__device__ __forceinline__ void chunk_gates(float* sm, float* misc, const float* ga,
                                            const float* be, int len, int l) {
  constexpr int TPL = C / kWave;
  float G[TPL];
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < TPL; ++r) s += ga[r];
  const float excl = wave_incl_scan(s) - s;
  float run = excl;
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    run += ga[r];
    G[r] = run;
  }
  const int tl = len - 1;
  float glast = G[0];
#pragma unroll
  for (int r = 1; r < TPL; ++r)
    if ((tl % TPL) == r) glast = G[r];
  glast = __shfl(glast, tl / TPL, kWave);
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    const int t = TPL * l + r;
    sm[t] = G[r];
    sm[C + t] = __expf(G[r]);
    sm[2 * C + t] = be[r];
    sm[3 * C + t] = t < len ? __expf(glast - G[r]) : 0.f;
  }
  if (l == 0) *misc = __expf(glast);
}

// The u-th lower-triangular 16 x 16 tile (ti >= tj) handled by wave w.  With NT = 2 NW,
// wave w takes block rows w and NT - 1 - w (NT + 1 tiles for every wave); otherwise tiles
// are dealt round-robin in row-major order.  Closed form, so tile loops stay branch-free.
template <int NT, int NW>
__device__ __forceinline__ void lower_tile(int w, int u, int& ti, int& tj) {
  if constexpr (NT == 2 * NW) {
    const bool first = u <= w;
    ti = first ? w : NT - 1 - w;
    tj = first ? u : u - (w + 1);
  } else {
    const int idx = w + NW * u;
    int i = (int)((__builtin_sqrtf(8.f * (float)idx + 1.f) - 1.f) * 0.5f);
    i += ((i + 1) * (i + 2) / 2 <= idx) ? 1 : 0;
    i -= (i * (i + 1) / 2 > idx) ? 1 : 0;
    ti = i;
    tj = idx - i * (i + 1) / 2;
  }
}

// Whether wave w has a u-th tile.
template <int NT, int NW>
__device__ __forceinline__ bool has_tile(int w, int u) {
  constexpr int NLOW = NT * (NT + 1) / 2;
  if constexpr (NT == 2 * NW || NLOW % NW == 0) return true;
  return w + NW * u < NLOW;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)b) << 16);
}

template <int D, int C, int NJ_>
__global__ __launch_bounds__(D * 4 / NJ_) void k_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const void* __restrict__ beta, int beta_f32,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, bf16* __restrict__ o,
    float* __restrict__ ht, int T, int Ttot, int H, int Hg, float scale) {
  typedef FusedCfg<D, C, NJ_> F;
  constexpr int NT = F::NT, NDK = F::NDK, NJ = F::NJ, LDC = F::LDC, LDT = F::LDT,
                TPL = F::TPL, CPR = F::CPR;
  const int n = blockIdx.x / H, h = blockIdx.x - n * H;
  const int hk = h / (H / Hg);
  const long qstride = (long)Hg * D, vstride = (long)H * D;
  const bf16* qh = q + (long)hk * D;
  const bf16* kh = k + (long)hk * D;
  const bf16* vh = v + (long)h * D;

  extern __shared__ __align__(16) char smem[];
  bf16* S0 = reinterpret_cast<bf16*>(smem);
  bf16* S1 = S0 + F::SLAB;
  bf16* S2 = S1 + F::SLAB;
  bf16* S3 = S2 + F::SLAB;
  float* sGates = reinterpret_cast<float*>(S3 + F::KT);  // [2][4][C]
  float* sMisc = sGates + F::GATES;                       // [2]: e^{G_last}
  float* sAd = sMisc + 2;
  f16* A16 = reinterpret_cast<f16*>(S0);

  int cs0, L;
  seq_span(cu, n, T, Ttot, cs0, L);
  const int nchunks = (L + C - 1) / C;

  // State: st[j][db] holds rows dk = 16 db + 4 (l/16) + e of column
  // 16 NJ w + NJ (l%16) + j.
  f32x4 st[NJ][NDK];
  const long hoff = ((long)n * H + h) * D * D;
  {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 16 * NJ * w + NJ * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int db = 0; db < NDK; ++db) st[j][db] = zero4();
    if (h0) {
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            st[j][db][e] = h0[hoff + (long)(16 * db + g4 + e) * D + dv0 + j];
    }
  }
  // bf16 copy of the state in the B-operand form of the K h, Q h products, refreshed once
  // per chunk after the state update.
  bf16x4 stb[NJ][NDK];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int db = 0; db < NDK; ++db) stb[j][db] = __builtin_convertvector(st[j][db], bf16x4);

  float pg[TPL], pb[TPL];
  if (nchunks > 0) {
    const int len0 = min(C, L), l = lane_id(), w = wave_id();
    dma_tile<F, D>(S0, kh + (long)cs0 * qstride, qstride, len0, w, l);
    dma_tile<F, D>(S1, qh + (long)cs0 * qstride, qstride, len0, w, l);
    dma_tile<F, D>(S2, vh + (long)cs0 * vstride, vstride, len0, w, l);
    if (w == 0) {
      load_gates<C>(pg, pb, g, beta, beta_f32, cs0, len0, h, H, l);
      chunk_gates<C>(sGates, sMisc, pg, pb, len0, l);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies have landed
    if (len0 < C) {
      __syncthreads();
      zero_tail<F, C>(S0, len0, threadIdx.x);
      zero_tail<F, C>(S1, len0, threadIdx.x);
      zero_tail<F, C>(S2, len0, threadIdx.x);
    }
  }
  __syncthreads();

  for (int m = 0; m < nchunks; ++m) {
    const int cs = cs0 + m * C;
    const int len = min(C, L - m * C);
    const int buf = m & 1;
    const float* sG = sGates + buf * 4 * C;
    const float* sEG = sG + C;
    const float* sB = sG + 2 * C;
    const float* sDec = sG + 3 * C;
    // Lane / wave / thread ids are re-derived opaquely at every phase, so the compiler
    // computes each phase's many LDS addresses inside that phase instead of holding them
    // in registers across the chunk.
    int tid, l, w, g4, dvl;
    auto phase = [&]() {
      tid = threadIdx.x;
      opaque(tid);
      l = tid & 63;
      w = __builtin_amdgcn_readfirstlane(tid >> 6);
      g4 = 4 * (l >> 4);
      dvl = 16 * NJ * w + NJ * (l & 15);  // this lane's first state column
    };
    phase();

    // (A) K^T scaled by e^{G_last - G} (the weight the state update gives v_new) into S3,
    // from the K tile in S0; token pairs are packed into 4-byte writes.
    for (int i = tid; i < (C / 2) * CPR; i += F::NTH) {
      const int tp = i / CPR, c8 = (i - tp * CPR) * 8, t = 2 * tp;
      const float d0 = sDec[t], d1 = sDec[t + 1];
      union {
        uint4 u;
        bf16 e[8];
      } k0, k1;
      k0.u = *reinterpret_cast<const uint4*>(S0 + swz<D>(t, c8));
      k1.u = *reinterpret_cast<const uint4*>(S0 + swz<D>(t + 1, c8));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(S3 + (c8 + e) * LDT + t) =
            pack2(d0 * (float)k0.e[e], d1 * (float)k1.e[e]);
    }

    phase();
    // (D1) K Q^T lower tiles (transposed orientation: rows j, columns i) and
    // R = beta (V - e^G K h) for this wave's columns, kept as the bf16 operand it becomes.
    f32x4 pacc[F::MAXT];
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      pacc[u] = zero4();
      if (has_tile<NT, F::NW>(w, u)) {
        int ti, tj;
        lower_tile<NT, F::NW>(w, u, ti, tj);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          pacc[u] = Mma<bf16>::mma(frag_swz<D>(S0, tj * 16, 32 * kk, l),
                                   frag_swz<D>(S1, ti * 16, 32 * kk, l), pacc[u]);
      }
      sched_fence();
    }
    bf16x4 R[NT][NJ];
    {
      ARow<bf16, NDK / 2> a[2];
      load_arow_swz<D, NDK / 2>(a[0], S0, 0, l);
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (tb + 1 < NT) load_arow_swz<D, NDK / 2>(a[(tb + 1) & 1], S0, (tb + 1) * 16, l);
        sched_fence();
        f32x4 x[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) x[j] = zero4();
        mma_arow<bf16, NDK / 2, NJ, 1, NDK, 1>(x, a[tb & 1], &stb[0][0], NDK);
        const f32x4 eg = *reinterpret_cast<const f32x4*>(sEG + tb * 16 + g4);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(sB + tb * 16 + g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = tb * 16 + g4 + e;
          const bf16* vp = S2 + swz<D>(t, dvl);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            R[tb][j][e] = (bf16)(bt[e] * ((float)vp[j] - eg[e] * x[j][e]));
        }
        sched_fence();
      }
    }
    __syncthreads();  // V consumed; K^T written

    phase();
    // (D2) P -> S2 (bf16); K K^T lower tiles.
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      if (has_tile<NT, F::NW>(w, u)) {
        int ti, tj;
        lower_tile<NT, F::NW>(w, u, ti, tj);
        const int i = ti * 16 + (l & 15);
        const int j0 = tj * 16 + g4;
        const float Gi = sG[i];
        const f32x4 Gj = *reinterpret_cast<const f32x4*>(sG + j0);
        bf16x4 pv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dec = __expf(fminf(Gi - Gj[e], 0.f));
          pv4[e] = (bf16)((i >= j0 + e) ? dec * pacc[u][e] : 0.f);
        }
        *reinterpret_cast<bf16x4*>(S2 + i * LDC + j0) = pv4;
      }
    }
    f32x4 aacc[F::MAXT];
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      aacc[u] = zero4();
      if (has_tile<NT, F::NW>(w, u)) {
        int ti, tj;
        lower_tile<NT, F::NW>(w, u, ti, tj);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          aacc[u] = Mma<bf16>::mma(frag_swz<D>(S0, tj * 16, 32 * kk, l),
                                   frag_swz<D>(S0, ti * 16, 32 * kk, l), aacc[u]);
      }
      sched_fence();
    }
    __syncthreads();  // K consumed

    phase();
    // (E) A -> S0 (fp16; diagonal blocks fp32 in sAd).
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      if (has_tile<NT, F::NW>(w, u)) {
        int ti, tj;
        lower_tile<NT, F::NW>(w, u, ti, tj);
        const int i = ti * 16 + (l & 15);
        const int j0 = tj * 16 + g4;
        const float Gi = sG[i], bi = sB[i];
        const f32x4 Gj = *reinterpret_cast<const f32x4*>(sG + j0);
        f32x4 a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dec = __expf(fminf(Gi - Gj[e], 0.f));
          a4[e] = (i > j0 + e) ? bi * dec * aacc[u][e] : 0.f;
        }
        if (ti == tj) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sAd[ti * 16 * kAdLd + (i & 15) * kAdLd + ((j0 + e) & 15)] = a4[e];
        } else {
          *reinterpret_cast<f16x4*>(A16 + i * LDC + j0) = __builtin_convertvector(a4, f16x4);
        }
      }
    }
    __syncthreads();  // A written

    phase();
    // (F) T = (I + A)^-1 in place over A (fp16), then to bf16 with the T^T half zeroed, so
    // S0 holds exactly the lower-triangular T.
    solve_tril<F::NW, C, f16, true>(A16, LDC, sAd, A16, LDC, tid, w, l);
    for (int i = tid; i < C * (C / 8); i += F::NTH) {
      const int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
      const f16x8 hv = *reinterpret_cast<const f16x8*>(A16 + r * LDC + c8);
      f32x8 fv = __builtin_convertvector(hv, f32x8);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c8 + e > r) fv[e] = 0.f;
      *reinterpret_cast<bf16x8*>(S0 + r * LDC + c8) = __builtin_convertvector(fv, bf16x8);
    }
    __syncthreads();

    phase();
    // (G) v_new = T R, kept as its bf16 operand form (T lower: row block tb needs k < 16 (tb+1)).
    bf16x4 vn[NT][NJ];
    {
      ARow<bf16, NT / 2> a[2];
      load_arow<bf16, NT / 2>(a[0], S0, LDC, 0, 0, 1, l);
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (tb + 1 < NT) load_arow<bf16, NT / 2>(a[(tb + 1) & 1], S0, LDC, (tb + 1) * 16, 0, tb + 2, l);
        sched_fence();
        f32x4 acc[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = zero4();
        mma_arow<bf16, NT / 2, NJ, 1, 1, NJ>(acc, a[tb & 1], &R[0][0], tb + 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) vn[tb][j] = __builtin_convertvector(acc[j], bf16x4);
        sched_fence();
      }
    }
    const bool more = m + 1 < nchunks;
    const int csn = cs + C, lenn = min(C, L - (m + 1) * C);
    if (more && w == 0) load_gates<C>(pg, pb, g, beta, beta_f32, csn, lenn, h, H, l);
    __syncthreads();  // T no longer read
    // Next chunk's K straight into S0.
    if (more) dma_tile<F, D>(S0, kh + (long)csn * qstride, qstride, lenn, w, l);

    phase();
    // (H) o = scale (e^G Q h + P v_new) for this wave's columns, one token block at a time.
    {
      ARow<bf16, NDK / 2> aq[2];
      ARow<bf16, NT / 2> ap[2];
      load_arow_swz<D, NDK / 2>(aq[0], S1, 0, l);
      load_arow<bf16, NT / 2>(ap[0], S2, LDC, 0, 0, 1, l);
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (tb + 1 < NT) {
          load_arow_swz<D, NDK / 2>(aq[(tb + 1) & 1], S1, (tb + 1) * 16, l);
          load_arow<bf16, NT / 2>(ap[(tb + 1) & 1], S2, LDC, (tb + 1) * 16, 0, tb + 2, l);
        }
        sched_fence();
        f32x4 y[NJ], z[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) y[j] = z[j] = zero4();
        mma_arow<bf16, NDK / 2, NJ, 1, NDK, 1>(y, aq[tb & 1], &stb[0][0], NDK);
        mma_arow<bf16, NT / 2, NJ, 1, 1, NJ>(z, ap[tb & 1], &vn[0][0], tb + 1);
        const f32x4 eg = *reinterpret_cast<const f32x4*>(sEG + tb * 16 + g4);
        bf16* op = o + ((long)(cs + tb * 16 + g4) * H + h) * D + dvl;
        const long ostride = (long)H * D;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // full chunks store unconditionally (a uniform branch); a partial last chunk
          // stores its valid rows only
          if (len == C || tb * 16 + g4 + e < len) {
            if constexpr (NJ == 2) {
              bf16x2_t ov;
              ov[0] = (bf16)(scale * fmaf(eg[e], y[0][e], z[0][e]));
              ov[1] = (bf16)(scale * fmaf(eg[e], y[1][e], z[1][e]));
              *reinterpret_cast<bf16x2_t*>(op + e * ostride) = ov;
            } else {
              op[e * ostride] = (bf16)(scale * fmaf(eg[e], y[0][e], z[0][e]));
            }
          }
        }
        sched_fence();
      }
    }
    __syncthreads();  // Q and P no longer read
    // Next chunk's Q and V straight into S1 and S2.
    if (more) {
      dma_tile<F, D>(S1, qh + (long)csn * qstride, qstride, lenn, w, l);
      dma_tile<F, D>(S2, vh + (long)csn * vstride, vstride, lenn, w, l);
    }

    phase();
    // (I) h = e^{G_last} h + (K e^{G_last - G})^T v_new, then refresh the bf16 copy.
    {
      const float eglast = sMisc[buf];
      ARow<bf16, NT / 2> a[2];
      load_arow<bf16, NT / 2>(a[0], S3, LDT, 0, 0, NT, l);
#pragma unroll
      for (int db = 0; db < NDK; ++db) {
        if (db + 1 < NDK) load_arow<bf16, NT / 2>(a[(db + 1) & 1], S3, LDT, (db + 1) * 16, 0, NT, l);
        sched_fence();
#pragma unroll
        for (int j = 0; j < NJ; ++j) st[j][db] *= eglast;
        mma_arow<bf16, NT / 2, NJ, NDK, 1, NJ>(&st[0][db], a[db & 1], &vn[0][0], NT);
        sched_fence();
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int db = 0; db < NDK; ++db) stb[j][db] = __builtin_convertvector(st[j][db], bf16x4);
    }
    if (more) {
      if (w == 0) chunk_gates<C>(sGates + (buf ^ 1) * 4 * C, sMisc + (buf ^ 1), pg, pb, lenn, l);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next chunk's copies have landed
      if (lenn < C) {
        __syncthreads();
        zero_tail<F, C>(S0, lenn, tid);
        zero_tail<F, C>(S1, lenn, tid);
        zero_tail<F, C>(S2, lenn, tid);
      }
    }
    __syncthreads();  // next chunk's tiles and gates visible; this chunk's reads done
  }

  if (ht) {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 16 * NJ * w + NJ * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          ht[hoff + (long)(16 * db + g4 + e) * D + dv0 + j] = st[j][db][e];
  }
}

template <int D, int C>
hipError_t run_fused(const Problem& p, hipStream_t st) {
  constexpr int NJ = kFusedNJ;
  typedef FusedCfg<D, C, NJ> F;
  const size_t sm = F::lds_bytes();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_fused<D, C, NJ>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const int grid = p.N * p.H;
  if (grid == 0) return hipSuccess;
  k_fused<D, C, NJ><<<grid, F::NTH, sm, st>>>(
      static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), static_cast<const bf16*>(p.v),
      p.g, p.beta, p.beta_f32 ? 1 : 0, p.h0, p.cu, static_cast<bf16*>(p.o), p.ht, p.T, p.Ttot,
      p.H, p.Hg, p.scale);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(const Problem& p) { return !p.f32 && (p.D == 64 || p.D == 128); }

hipError_t launch_fused(const Problem& p, hipStream_t st) {
  if (p.D == 64) return p.C == 64 ? run_fused<64, 64>(p, st) : run_fused<64, 128>(p, st);
  return p.C == 64 ? run_fused<128, 64>(p, st) : run_fused<128, 128>(p, st);
}

}  // namespace gdn
