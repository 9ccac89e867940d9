// Fused single-launch chunked Gated DeltaNet forward (the megakernel idea of the
// MegaGDN-PTO page, sections 1.3 and 4.5: all seven stages in one launch, intermediates
// kept on chip), designed for gfx950.
//
// One workgroup owns one (sequence, value head) and walks its chunks in order; nothing
// crosses workgroups, so no grid barrier is needed (the page's all-core SyncAll barrier
// has no counterpart here).  D/16 waves; wave w owns state columns [16w, 16w+16) for all
// Dk rows as fp32 accumulator tiles, so the recurrent chain K h -> R -> T R -> (o, h)
// never leaves registers.  Per chunk, with G the in-chunk prefix sum of g:
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
// LDS: four C x (D|C) bf16 slabs, re-used by phase —
//   S0: K            -> A (fp16, off-diagonal blocks) for the solve
//   S1: Q            -> P = gated, masked Q K^T (bf16)
//   S2: V            -> M = T / T^T (fp16 during the solve, then bf16)
//   S3: K^T
// plus G, e^G, beta, e^{G_last-G} and the fp32 diagonal blocks of A.  The next chunk's
// q, k, v, g, beta are loaded into registers while the current chunk computes.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_solve.h"

namespace gdn {

namespace {

template <int D, int C>
struct FusedCfg {
  static constexpr int NW = D / 16;
  static constexpr int NTH = NW * kWave;  // = 4 D (the launch bound)
  static constexpr int NT = C / 16;   // token blocks per chunk
  static constexpr int NDK = D / 16;  // key blocks
  static constexpr int LDD = D + 8;   // row of a [C][D] bf16 operand
  static constexpr int LDC = C + 8;   // row of a [*][C] 16-bit operand
  static constexpr int SLAB = (C * LDD > C * LDC ? C * LDD : C * LDC);  // elements
  static constexpr int KT = D * LDC;
  static constexpr int NP = C / 32;  // 16-byte pieces per thread per q/k/v tile
  static constexpr int NLOW = NT * (NT + 1) / 2;
  static constexpr int MAXT = (NLOW + NW - 1) / NW;
  static constexpr size_t lds_bytes() {
    return (size_t)(3 * SLAB + KT) * 2 + (size_t)4 * C * 4 + (size_t)(C / 16) * 16 * kAdLd * 4 +
           16;
  }
};

template <int D, int C>
struct Prefetch {
  uint4 q[FusedCfg<D, C>::NP], k[FusedCfg<D, C>::NP], v[FusedCfg<D, C>::NP];
  float g, b;
};

template <int D, int C>
__device__ __forceinline__ void prefetch(Prefetch<D, C>& pf, const bf16* q, const bf16* k,
                                         const bf16* v, const float* g, const void* beta,
                                         int beta_f32, int cs, int len, int h, int hk, int H,
                                         int Hg) {
  typedef FusedCfg<D, C> F;
  constexpr int PPR = D / 8;  // pieces per row
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < F::NP; ++r) {
    const int pc = tid + r * F::NTH;
    const int t = pc / PPR, cp = pc - t * PPR;
    const uint4 z = make_uint4(0, 0, 0, 0);
    pf.q[r] = z;
    pf.k[r] = z;
    pf.v[r] = z;
    if (t < len) {
      const long qk = ((long)(cs + t) * Hg + hk) * D + cp * 8;
      const long vo = ((long)(cs + t) * H + h) * D + cp * 8;
      pf.q[r] = *reinterpret_cast<const uint4*>(q + qk);
      pf.k[r] = *reinterpret_cast<const uint4*>(k + qk);
      pf.v[r] = *reinterpret_cast<const uint4*>(v + vo);
    }
  }
  pf.g = 0.f;
  pf.b = 0.f;
  if (tid < len) {
    const long gi = (long)(cs + tid) * H + h;
    pf.g = g[gi];
    pf.b = load_beta(beta, beta_f32, gi);
  }
}

// Lower-triangular tile u (row-major enumeration of ti >= tj) -> (ti, tj).
__device__ __forceinline__ void lower_tile(int u, int& ti, int& tj) {
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= u) ++i;
  ti = i;
  tj = u - i * (i + 1) / 2;
}

template <int D, int C>
__global__ __launch_bounds__(D * 4) void k_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const void* __restrict__ beta, int beta_f32,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, bf16* __restrict__ o,
    float* __restrict__ ht, int T, int Ttot, int H, int Hg, float scale) {
  typedef FusedCfg<D, C> F;
  constexpr int NT = F::NT, NDK = F::NDK, LDD = F::LDD, LDC = F::LDC;
  const int n = blockIdx.x / H, h = blockIdx.x - n * H;
  const int hk = h / (H / Hg);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int dv = 16 * w + (l & 15);   // this lane's state / output column
  const int g4 = 4 * (l >> 4);

  extern __shared__ __align__(16) char smem[];
  bf16* S0 = reinterpret_cast<bf16*>(smem);
  bf16* S1 = S0 + F::SLAB;
  bf16* S2 = S1 + F::SLAB;
  bf16* S3 = S2 + F::SLAB;
  float* sG = reinterpret_cast<float*>(S3 + F::KT);
  float* sEG = sG + C;
  float* sB = sEG + C;
  float* sDec = sB + C;
  float* sAd = sDec + C;
  float* sMisc = sAd + (C / 16) * 16 * kAdLd;
  f16* A16 = reinterpret_cast<f16*>(S0);
  f16* M16 = reinterpret_cast<f16*>(S2);

  int cs0, L;
  seq_span(cu, n, T, Ttot, cs0, L);
  const int nchunks = (L + C - 1) / C;

  // State tiles: st[db] holds rows dk = 16 db + g4 + e of column dv.
  f32x4 st[NDK];
  const long hoff = ((long)n * H + h) * D * D;
#pragma unroll
  for (int db = 0; db < NDK; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) st[db][e] = h0 ? h0[hoff + (long)(16 * db + g4 + e) * D + dv] : 0.f;

  Prefetch<D, C> pf;
  if (nchunks > 0) prefetch<D, C>(pf, q, k, v, g, beta, beta_f32, cs0, min(C, L), h, hk, H, Hg);

  for (int m = 0; m < nchunks; ++m) {
    const int cs = cs0 + m * C;
    const int len = min(C, L - m * C);

    // (A) registers -> LDS: K, Q, V row-major, K^T, raw g and beta.
    {
      constexpr int PPR = D / 8;
#pragma unroll
      for (int r = 0; r < F::NP; ++r) {
        const int pc = tid + r * F::NTH;
        const int t = pc / PPR, c8 = (pc - t * PPR) * 8;
        *reinterpret_cast<uint4*>(S0 + t * LDD + c8) = pf.k[r];
        *reinterpret_cast<uint4*>(S1 + t * LDD + c8) = pf.q[r];
        *reinterpret_cast<uint4*>(S2 + t * LDD + c8) = pf.v[r];
        union {
          uint4 u;
          bf16 e[8];
        } kk;
        kk.u = pf.k[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) S3[(c8 + e) * LDC + t] = kk.e[e];
      }
      if (tid < C) {
        sG[tid] = pf.g;
        sB[tid] = pf.b;
      }
    }
    // (B) start loading the next chunk.
    if (m + 1 < nchunks)
      prefetch<D, C>(pf, q, k, v, g, beta, beta_f32, cs + C, min(C, L - (m + 1) * C), h, hk,
                     H, Hg);
    __syncthreads();

    // (C) wave 0: G = prefix sum of g, e^G, e^{G_last - G}, e^{G_last}.
    if (w == 0) {
      if constexpr (C == 128) {
        const float a = sG[2 * l], b = sG[2 * l + 1];
        const float incl = wave_incl_scan(a + b);
        sG[2 * l] = incl - b;
        sG[2 * l + 1] = incl;
      } else {
        sG[l] = wave_incl_scan(sG[l]);
      }
      const float glast = sG[len - 1];
#pragma unroll
      for (int r = 0; r < C / kWave; ++r) {
        const int t = l + r * kWave;
        const float G = sG[t];
        sEG[t] = __expf(G);
        sDec[t] = t < len ? __expf(glast - G) : 0.f;
      }
      if (l == 0) sMisc[0] = __expf(glast);
    }

    // (D) matrix-core phase 1: K K^T and K Q^T lower tiles (transposed orientation), and
    // X = K h, Y = Q h for this wave's columns.
    f32x4 aacc[F::MAXT], pacc[F::MAXT];
#pragma unroll
    for (int u = 0; u < F::MAXT; ++u) {
      aacc[u] = zero4();
      pacc[u] = zero4();
      const int idx = w + F::NW * u;
      if (idx < F::NLOW) {
        int ti, tj;
        lower_tile(idx, ti, tj);
        mma_lds<bf16>(aacc[u], S0, LDD, tj * 16, S0, LDD, ti * 16, 0, D);
        mma_lds<bf16>(pacc[u], S0, LDD, tj * 16, S1, LDD, ti * 16, 0, D);
      }
    }
    f32x4 x[NT], y[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      x[tb] = zero4();
      y[tb] = zero4();
      mma_accB<bf16, NDK>(x[tb], S0, LDD, tb * 16, 0, st, NDK);
      mma_accB<bf16, NDK>(y[tb], S1, LDD, tb * 16, 0, st, NDK);
    }
    __syncthreads();  // K, Q no longer read; G ready

    // (E) epilogues: A -> S0 (fp16) / sAd (fp32 diagonal blocks), P -> S1 (bf16),
    // R = beta (V - e^G X) in registers (V read from S2), Y *= e^G.
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
        bf16x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e;
          const float dec = (i >= j) ? __expf(Gi - sG[j]) : 0.f;
          const float a = (i > j) ? bi * dec * aacc[u][e] : 0.f;
          av[e] = (f16)a;
          pv[e] = (bf16)(dec * pacc[u][e]);
          if (ti == tj) sAd[ti * 16 * kAdLd + (i & 15) * kAdLd + (j & 15)] = a;
        }
        if (ti != tj) *reinterpret_cast<f16x4*>(A16 + i * LDC + j0) = av;
        *reinterpret_cast<bf16x4*>(S1 + i * LDC + j0) = pv;
      }
    }
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + g4 + e;
        const float vv = (float)S2[t * LDD + dv];
        const float eg = sEG[t];
        x[tb][e] = sB[t] * (vv - eg * x[tb][e]);
        y[tb][e] *= eg;
      }
    __syncthreads();  // A, P written; V consumed

    // (F) T = (I + A)^-1 into S2 (fp16), then to bf16 in place.
    solve_tril<F::NW, C, f16>(A16, LDC, sAd, M16, LDC);
    for (int i = tid; i < C * (C / 8); i += F::NTH) {
      const int r = i / (C / 8), c8 = (i - r * (C / 8)) * 8;
      const f16x8 hv = *reinterpret_cast<const f16x8*>(M16 + r * LDC + c8);
      const f32x8 fv = __builtin_convertvector(hv, f32x8);
      *reinterpret_cast<bf16x8*>(S2 + r * LDC + c8) = __builtin_convertvector(fv, bf16x8);
    }
    __syncthreads();

    // (G) v_new = T R (T lower: mask M's upper half).
    f32x4 vn[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      vn[tb] = zero4();
      mma_accB<bf16, NT, true>(vn[tb], S2, LDC, tb * 16, 0, x, tb + 1, 0);
    }
    // (H) o = scale (Y + P v_new) for this wave's columns.
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      mma_accB<bf16, NT>(y[tb], S1, LDC, tb * 16, 0, vn, tb + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + g4 + e;
        if (t < len) o[((long)(cs + t) * H + h) * D + dv] = (bf16)(scale * y[tb][e]);
      }
    }
    // (I) h = e^{G_last} h + K^T (e^{G_last - G} v_new).
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) vn[tb][e] *= sDec[tb * 16 + g4 + e];
    const float eglast = sMisc[0];
#pragma unroll
    for (int db = 0; db < NDK; ++db) {
      st[db] *= eglast;
      mma_accB<bf16, NT>(st[db], S3, LDC, db * 16, 0, vn, NT);
    }
    __syncthreads();  // all LDS reads of this chunk done before the next chunk's writes
  }

  if (ht) {
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) ht[hoff + (long)(16 * db + g4 + e) * D + dv] = st[db][e];
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
