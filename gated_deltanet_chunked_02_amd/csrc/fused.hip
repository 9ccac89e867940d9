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
// LDS: four bf16 slabs re-used by phase —
//   S0: K            -> A (fp16, off-diagonal blocks) for the solve
//   S1: Q            -> M = T / T^T (fp16 during the solve, then bf16)
//   S2: V            -> P = gated, masked Q K^T (bf16)
//   S3: K^T scaled by e^{G_last - G}
// plus the fp32 diagonal blocks of A and the chunk's gate vectors (G, e^G, beta,
// e^{G_last-G}), which wave 0 computes for the next chunk at the end of the current one
// (double-buffered).  The next chunk's k, v (then q, g, beta) are loaded into registers
// during the second half of the current chunk.  R and v_new live in registers in the
// bf16 form in which they feed the matrix cores.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_solve.h"

namespace gdn {

namespace {

template <int D, int C>
struct FusedCfg {
  static constexpr int NJ = 2;            // 16-column blocks per wave
  static constexpr int NW = D / 32;       // waves
  static constexpr int NTH = NW * kWave;  // = 2 D (the launch bound)
  static constexpr int NT = C / 16;       // token blocks per chunk
  static constexpr int NDK = D / 16;      // key blocks
  static constexpr int LDD = D + 8;       // row of a [C][D] bf16 operand
  static constexpr int LDC = C + 8;       // row of a [*][C] 16-bit operand
  static constexpr int LDT = C + 12;      // row of K^T (8-byte reads; spreads the writes)
  static constexpr int SLAB = (C * LDD > C * LDC ? C * LDD : C * LDC);  // elements
  static constexpr int KT = D * LDT;
  static constexpr int PPR = D / 8;            // 16-byte pieces per q/k/v row
  static constexpr int RG = NTH / PPR;         // row groups covered by one pass
  static constexpr int NP = C * PPR / NTH;     // pieces per thread per tile (even)
  static constexpr int NLOW = NT * (NT + 1) / 2;
  static constexpr int MAXT = (NLOW + NW - 1) / NW;
  static constexpr int TPL = C / kWave;        // tokens per lane in the gate scan
  static_assert(NP % 2 == 0, "pieces come in token pairs");
  // Per-chunk gate vectors, double-buffered: [2][4][C] = G, e^G, beta, e^{G_last - G}.
  static constexpr int GATES = 2 * 4 * C;
  static constexpr size_t lds_bytes() {
    return (size_t)(3 * SLAB + KT) * 2 + (size_t)GATES * 4 + 2 * 4 +
           (size_t)(C / 16) * 16 * kAdLd * 4 + 8;
  }
};

// Token of piece r of a thread in row group rg: pieces come in (even, odd) token pairs.
template <int D, int C>
__device__ __forceinline__ int piece_row(int rg, int r) {
  typedef FusedCfg<D, C> F;
  return 2 * (rg + (r >> 1) * F::RG) + (r & 1);
}

template <int D, int C>
__device__ __forceinline__ void load_pieces(uint4* dst, const bf16* src, long tok_stride,
                                            int cs, int len, int tid) {
  typedef FusedCfg<D, C> F;
  const int rg = tid / F::PPR, cp = tid - rg * F::PPR;
#pragma unroll
  for (int r = 0; r < F::NP; ++r) {
    const int t = piece_row<D, C>(rg, r);
    dst[r] = make_uint4(0, 0, 0, 0);
    if (t < len)
      dst[r] = *reinterpret_cast<const uint4*>(src + (long)(cs + t) * tok_stride + cp * 8);
  }
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

// Lower-triangular tile u (row-major enumeration of ti >= tj) -> (ti, tj).
__device__ __forceinline__ void lower_tile(int u, int& ti, int& tj) {
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= u) ++i;
  ti = i;
  tj = u - i * (i + 1) / 2;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)b) << 16);
}

template <int D, int C>
__global__ __launch_bounds__(D * 2) void k_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const void* __restrict__ beta, int beta_f32,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, bf16* __restrict__ o,
    float* __restrict__ ht, int T, int Ttot, int H, int Hg, float scale) {
  typedef FusedCfg<D, C> F;
  constexpr int NT = F::NT, NDK = F::NDK, NJ = F::NJ, LDD = F::LDD, LDC = F::LDC,
                LDT = F::LDT, TPL = F::TPL;
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
  f16* M16 = reinterpret_cast<f16*>(S1);

  int cs0, L;
  seq_span(cu, n, T, Ttot, cs0, L);
  const int nchunks = (L + C - 1) / C;

  // State: st[j][db] holds rows dk = 16 db + 4 (l/16) + e of column 32 w + 2 (l%16) + j.
  f32x4 st[NJ][NDK];
  const long hoff = ((long)n * H + h) * D * D;
  {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 32 * w + 2 * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int db = 0; db < NDK; ++db) st[0][db] = st[1][db] = zero4();
    if (h0) {
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 hv =
              *reinterpret_cast<const float2*>(h0 + hoff + (long)(16 * db + g4 + e) * D + dv0);
          st[0][db][e] = hv.x;
          st[1][db][e] = hv.y;
        }
    }
  }

  uint4 pk[F::NP], pv[F::NP], pq[F::NP];
  float pg[TPL], pb[TPL];
  if (nchunks > 0) {
    const int len0 = min(C, L);
    load_pieces<D, C>(pk, kh, qstride, cs0, len0, threadIdx.x);
    load_pieces<D, C>(pv, vh, vstride, cs0, len0, threadIdx.x);
    load_pieces<D, C>(pq, qh, qstride, cs0, len0, threadIdx.x);
    if (wave_id() == 0) {
      load_gates<C>(pg, pb, g, beta, beta_f32, cs0, len0, h, H, lane_id());
      chunk_gates<C>(sGates, sMisc, pg, pb, len0, lane_id());
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
    // Lane / wave / thread ids are re-derived opaquely each chunk so the compiler keeps
    // the many derived LDS addresses inside the loop instead of holding them in registers.
    int tid = threadIdx.x;
    opaque(tid);
    const int l = tid & 63, w = tid >> 6;
    const int g4 = 4 * (l >> 4);
    const int dvl = 32 * w + 2 * (l & 15);  // this lane's first state column

    // (A) registers -> LDS: K, Q, V row-major; K^T scaled by e^{G_last - G} (token pairs
    // packed), which is the weight the state update applies to v_new.
    {
      const int rg = tid / F::PPR, c8 = (tid - rg * F::PPR) * 8;
#pragma unroll
      for (int r = 0; r < F::NP; ++r) {
        const int t = piece_row<D, C>(rg, r);
        *reinterpret_cast<uint4*>(S0 + t * LDD + c8) = pk[r];
        *reinterpret_cast<uint4*>(S1 + t * LDD + c8) = pq[r];
        *reinterpret_cast<uint4*>(S2 + t * LDD + c8) = pv[r];
      }
#pragma unroll
      for (int r = 0; r < F::NP; r += 2) {
        const int t = piece_row<D, C>(rg, r);  // even; r + 1 holds token t + 1
        const float d0 = sDec[t], d1 = sDec[t + 1];
        union {
          uint4 u;
          bf16 e[8];
        } k0, k1;
        k0.u = pk[r];
        k1.u = pk[r + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint32_t*>(S3 + (c8 + e) * LDT + t) =
              pack2(d0 * (float)k0.e[e], d1 * (float)k1.e[e]);
      }
    }
    __syncthreads();

    // (D) K K^T and K Q^T lower tiles (transposed orientation) and X = K h for this wave's
    // columns; then R = beta (V - e^G X), kept as the bf16 operand it becomes.
    f32x4 aacc[F::MAXT], pacc[F::MAXT];
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      aacc[u] = zero4();
      pacc[u] = zero4();
      const int idx = w + F::NW * u;
      if (idx < F::NLOW) {
        int ti, tj;
        lower_tile(idx, ti, tj);
        mma_lds<bf16>(aacc[u], S0, LDD, tj * 16, S0, LDD, ti * 16, 0, D, l);
        mma_lds<bf16>(pacc[u], S0, LDD, tj * 16, S1, LDD, ti * 16, 0, D, l);
      }
    }
    bf16x4 R[NT][NJ];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      f32x4 x[NJ] = {zero4(), zero4()};
      mma_accB_n<bf16, NDK, NJ>(x, S0, LDD, tb * 16, 0, &st[0][0], NDK, 0, l);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + g4 + e;
        const bf16x2_t vv = *reinterpret_cast<const bf16x2_t*>(S2 + t * LDD + dvl);
        const float eg = sEG[t], bt = sB[t];
        R[tb][0][e] = (bf16)(bt * ((float)vv[0] - eg * x[0][e]));
        R[tb][1][e] = (bf16)(bt * ((float)vv[1] - eg * x[1][e]));
      }
    }
    __syncthreads();  // K and V no longer read

    // (E) A -> S0 (fp16; diagonal blocks fp32 in sAd), P -> S2 (bf16), then Y = e^G Q h.
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      const int idx = w + F::NW * u;
      if (idx < F::NLOW) {
        int ti, tj;
        lower_tile(idx, ti, tj);
        const int i = ti * 16 + (l & 15);
        const int j0 = tj * 16 + g4;
        const float Gi = sG[i], bi = sB[i];
        f16x4 av;
        bf16x4 pv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e;
          const float dec = (i >= j) ? __expf(Gi - sG[j]) : 0.f;
          const float a = (i > j) ? bi * dec * aacc[u][e] : 0.f;
          av[e] = (f16)a;
          pv4[e] = (bf16)(dec * pacc[u][e]);
          if (ti == tj) sAd[ti * 16 * kAdLd + (i & 15) * kAdLd + (j & 15)] = a;
        }
        if (ti != tj) *reinterpret_cast<f16x4*>(A16 + i * LDC + j0) = av;
        *reinterpret_cast<bf16x4*>(S2 + i * LDC + j0) = pv4;
      }
    }
    f32x4 y[NT][NJ];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      y[tb][0] = y[tb][1] = zero4();
      mma_accB_n<bf16, NDK, NJ>(y[tb], S1, LDD, tb * 16, 0, &st[0][0], NDK, 0, l);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float eg = sEG[tb * 16 + g4 + e];
        y[tb][0][e] *= eg;
        y[tb][1][e] *= eg;
      }
    }
    __syncthreads();  // A, P written; Q no longer read

    // (F) T = (I + A)^-1 into S1 (fp16), then to bf16 in place.
    solve_tril<F::NW, C, f16>(A16, LDC, sAd, M16, LDC, tid, w, l);
    for (int i = tid; i < C * (C / 8); i += F::NTH) {
      const int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
      const f16x8 hv = *reinterpret_cast<const f16x8*>(M16 + r * LDC + c8);
      const f32x8 fv = __builtin_convertvector(hv, f32x8);
      *reinterpret_cast<bf16x8*>(S1 + r * LDC + c8) = __builtin_convertvector(fv, bf16x8);
    }
    __syncthreads();

    // (G) v_new = T R (T lower: mask M's upper half), kept as its bf16 operand form.
    bf16x4 vn[NT][NJ];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      f32x4 acc[NJ] = {zero4(), zero4()};
      mma_accB_n<bf16, NT, NJ, true, 1, 1, NJ>(acc, S1, LDC, tb * 16, 0, &R[0][0], tb + 1, 0,
                                              l);
      vn[tb][0] = __builtin_convertvector(acc[0], bf16x4);
      vn[tb][1] = __builtin_convertvector(acc[1], bf16x4);
    }
    // Next chunk's K and V: issued here (R is dead), consumed at the top of the next chunk.
    const bool more = m + 1 < nchunks;
    const int csn = cs + C, lenn = min(C, L - (m + 1) * C);
    if (more) {
      load_pieces<D, C>(pk, kh, qstride, csn, lenn, tid);
      load_pieces<D, C>(pv, vh, vstride, csn, lenn, tid);
    }
    // (H) o = scale (Y + P v_new) for this wave's columns.
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      mma_accB_n<bf16, NT, NJ, false, 1, 1, NJ>(y[tb], S2, LDC, tb * 16, 0, &vn[0][0], tb + 1,
                                               0, l);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + g4 + e;
        if (t < len) {
          bf16x2_t ov;
          ov[0] = (bf16)(scale * y[tb][0][e]);
          ov[1] = (bf16)(scale * y[tb][1][e]);
          *reinterpret_cast<bf16x2_t*>(o + ((long)(cs + t) * H + h) * D + dvl) = ov;
        }
      }
    }
    if (more) {
      load_pieces<D, C>(pq, qh, qstride, csn, lenn, tid);
      if (w == 0) load_gates<C>(pg, pb, g, beta, beta_f32, csn, lenn, h, H, l);
    }
    // (I) h = e^{G_last} h + (K e^{G_last - G})^T v_new.
    const float eglast = sMisc[buf];
#pragma unroll
    for (int db = 0; db < NDK; ++db) {
      st[0][db] *= eglast;
      st[1][db] *= eglast;
      mma_accB_n<bf16, NT, NJ, false, NDK, 1, NJ>(&st[0][db], S3, LDT, db * 16, 0, &vn[0][0],
                                                  NT, 0, l);
    }
    if (more && w == 0)
      chunk_gates<C>(sGates + (buf ^ 1) * 4 * C, sMisc + (buf ^ 1), pg, pb, lenn, l);
    __syncthreads();  // all LDS reads of this chunk done before the next chunk's writes
  }

  if (ht) {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 32 * w + 2 * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<float2*>(ht + hoff + (long)(16 * db + g4 + e) * D + dv0) =
            make_float2(st[0][db][e], st[1][db][e]);
  }
}

template <int D, int C>
hipError_t run_fused(const Problem& p, hipStream_t st) {
  typedef FusedCfg<D, C> F;
  const size_t sm = F::lds_bytes();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_fused<D, C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const int grid = p.N * p.H;
  if (grid == 0) return hipSuccess;
  k_fused<D, C><<<grid, F::NTH, sm, st>>>(
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
