// The seven chunk stages as separate launches (the staged execution mode of the
// MegaGDN-PTO page, sections 1.1 and 7.4), written for gfx950.
//
//   stage 0  chunk table        cu_seqlens -> (sequence, first token, length, index)
//   stage 1  chunk_cumsum       G = in-chunk prefix sum of g            (page section 4.1)
//   stage 2  transpose          [T, H] -> [H, T] for G and beta         (page section 4.5)
//   stage 3  scaled_dot_kkt     A = beta_i e^{G_i-G_j} k_i.k_j, i > j    (page section 4.2)
//   stage 4  solve_tril         Tinv = (I + A)^-1                        (page section 4.4)
//   stage 5  wy_fast            U = Tinv diag(beta) V, W = Tinv diag(beta e^G) K (4.3)
//   stage 6  chunk_h            per chunk: h_c, v_new = U - W h_c,
//                               h <- e^{G_last} h + K^T (e^{G_last-G} v_new)
//                               (chunk_gated_delta_rule_fwd_h, TileLang x xLLM page)
//   stage 7  chunk_o            o = scale (diag(e^G) Q h_c + (Q K^T * e^{G_i-G_j})_{i>=j} v_new)
//
// Every chunk-parallel stage runs one 256-thread workgroup (4 waves) per (chunk, head);
// chunk_h runs one workgroup per (sequence, head, 64-column slice of the state).  Dense
// products use the 16x16 matrix-core tiles described in gdn_device.h.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_operands.h"
#include "gdn_solve.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T> struct Vec16 { static constexpr int n = 16 / (int)sizeof(T); };

__device__ __forceinline__ int4 load_chunk(const int32_t* table, int c) {
  return reinterpret_cast<const int4*>(table)[c];
}

// ------------------------------------------------------------------------- stage 0
// One workgroup of 1024 threads scans the chunk counts of all sequences (wave scans +
// a workgroup combine, repeated per 1024 sequences with a running carry).
__global__ __launch_bounds__(1024) void k_chunk_table(const int32_t* cu, int N, int T, int Ttot,
                                                      int C, int max_chunks, int32_t* table,
                                                      int32_t* seq_chunks) {
  __shared__ int s_part[16];
  // this block of sequences: each one's first chunk, first token and length
  __shared__ int s_off[1024], s_start[1024], s_len[1024];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  int4* tab = reinterpret_cast<int4*>(table);
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int start = 0, len = 0;
    if (n < N) seq_span(cu, n, T, Ttot, start, len);
    const int nc = (len + C - 1) / C;
    const int incl = wave_incl_scan_int(nc);
    if (l == kWave - 1) s_part[w] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
      const int x = s_part[i];
      wbase += (i < w) ? x : 0;
      total += x;
    }
    const int off = carry + wbase + incl - nc;
    if (n < N) seq_chunks[n] = min(off, max_chunks);
    s_off[tid] = off;  // past the block's sequences: the end (no chunk lies there)
    s_start[tid] = start;
    s_len[tid] = len;
    __syncthreads();
    // every thread writes rows of the table: row idx belongs to the last sequence of the
    // block whose first chunk is at or before idx (an empty sequence starts where the next
    // one does, so the search passes over it)
    const int cnt = min(1024, N - base);
    for (int idx = carry + tid; idx < min(carry + total, max_chunks); idx += 1024) {
      int lo = 0, hi = cnt - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= idx) lo = mid; else hi = mid - 1;
      }
      const int m = idx - s_off[lo];
      tab[idx] = make_int4(base + lo, s_start[lo] + m * C, min(C, s_len[lo] - m * C), m);
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) seq_chunks[N] = min(carry, max_chunks);
  for (int i = carry + tid; i < max_chunks; i += 1024) tab[i] = make_int4(0, 0, 0, 0);
}

// ------------------------------------------------------------------------- stage 1
// One workgroup per chunk.  The chunk's g block [len, H] is contiguous: stage it through
// LDS (coalesced), scan each head's column with one wave (C/64 tokens per lane), store back.
template <int C>
__global__ __launch_bounds__(kThreads) void k_cumsum(const int32_t* table, const float* g,
                                                     float* g_cum, int H) {
  const int4 ci = load_chunk(table, blockIdx.x);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  constexpr int HB = 64;
  __shared__ float tile[C][HB + 1];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  for (int hb = 0; hb < H; hb += HB) {
    const int nh = min(HB, H - hb);
    for (int i = tid; i < len * nh; i += kThreads) {
      const int t = i / nh, j = i - t * nh;
      tile[t][j] = g[(long)(start + t) * H + hb + j];
    }
    __syncthreads();
    for (int j = w; j < nh; j += kWaves) {
      if constexpr (C == 128) {
        const int t0 = 2 * l, t1 = 2 * l + 1;
        const float a = t0 < len ? tile[t0][j] : 0.f;
        const float b = t1 < len ? tile[t1][j] : 0.f;
        const float incl = wave_incl_scan(a + b);
        if (t0 < len) tile[t0][j] = incl - b;
        if (t1 < len) tile[t1][j] = incl;
      } else {
        const float a = l < len ? tile[l][j] : 0.f;
        const float incl = wave_incl_scan(a);
        if (l < len) tile[l][j] = incl;
      }
    }
    __syncthreads();
    for (int i = tid; i < len * nh; i += kThreads) {
      const int t = i / nh, j = i - t * nh;
      g_cum[(long)(start + t) * H + hb + j] = tile[t][j];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------- stage 2
// 64 x 64 tiles through LDS; both the read and the write side are row-contiguous.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_transpose(const T* in, T* out, int rows,
                                                        int cols) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += kThreads) {
    const int r = i >> 6, c = i & 63;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = in[(long)(r0 + r) * cols + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += kThreads) {
    const int c = i >> 6, r = i & 63;
    if (r0 + r < rows && c0 + c < cols) out[(long)(c0 + c) * rows + r0 + r] = tile[r][c];
  }
}

// Copy C rows of D elements (row stride `stride` elements in global memory) into a
// k-contiguous LDS matrix [C][ld]; rows >= rows_valid (>= 1) are zero.  16-byte pieces,
// up to eight loads in flight per thread: the loads are unconditional (rows past the end
// read the last valid row) and the zeroing is a select at the store.
template <typename T, int D, int C>
__device__ __forceinline__ void stage_rows(T* s, int ld, const T* src, long stride,
                                           int rows_valid) {
  constexpr int VE = Vec16<T>::n, VPR = D / VE, TOTAL = C * VPR;
  constexpr int ITER = (TOTAL + kThreads - 1) / kThreads, BATCH = ITER < 8 ? ITER : 8;
  static_assert(TOTAL % kThreads == 0 && ITER % BATCH == 0, "whole batches");
#pragma unroll
  for (int b0 = 0; b0 < ITER; b0 += BATCH) {
    uint4 val[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = threadIdx.x + (b0 + j) * kThreads;
      const int t = i / VPR, pc = i - t * VPR;
      val[j] = *reinterpret_cast<const uint4*>(src + min(t, rows_valid - 1) * stride + pc * VE);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = threadIdx.x + (b0 + j) * kThreads;
      const int t = i / VPR, pc = i - t * VPR;
      *reinterpret_cast<uint4*>(s + t * ld + pc * VE) =
          t < rows_valid ? val[j] : make_uint4(0, 0, 0, 0);
    }
  }
}

// Same source, stored transposed: s[d][t] = scale_t * src[t][d0 + d] for d < W columns.
template <typename T, int W, int C>
__device__ __forceinline__ void stage_rows_T(T* s, int ld, const T* src, long stride,
                                             int rows_valid, const float* scale_t) {
  constexpr int VE = Vec16<T>::n, VPR = W / VE, TOTAL = C * VPR;
  constexpr int ITER = (TOTAL + kThreads - 1) / kThreads, BATCH = ITER < 8 ? ITER : 8;
  static_assert(TOTAL % kThreads == 0 && ITER % BATCH == 0, "whole batches");
  union Piece {
    uint4 u;
    T e[VE];
  };
#pragma unroll
  for (int b0 = 0; b0 < ITER; b0 += BATCH) {
    Piece val[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = threadIdx.x + (b0 + j) * kThreads;
      const int t = i / VPR, pc = i - t * VPR;
      val[j].u = *reinterpret_cast<const uint4*>(src + min(t, rows_valid - 1) * stride + pc * VE);
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int i = threadIdx.x + (b0 + j) * kThreads;
      const int t = i / VPR, pc = i - t * VPR;
      const float f = t < rows_valid ? (scale_t ? scale_t[t] : 1.f) : 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) s[(pc * VE + e) * ld + t] = (T)(f * (float)val[j].e[e]);
    }
  }
}

// ------------------------------------------------------------------------- stage 3
template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_kkt(const int32_t* table, const TI* k,
                                                  const float* g_t, const void* beta_t,
                                                  int beta_f32, float* A, int Ttot, int H,
                                                  int Hg) {
  const int4 ci = load_chunk(table, blockIdx.x);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y, hk = h / (H / Hg);
  constexpr int LD = D + pad_of<TI>();
  extern __shared__ __align__(16) char smem[];
  TI* sK = reinterpret_cast<TI*>(smem);
  float* sG = reinterpret_cast<float*>(smem + C * LD * sizeof(TI));
  float* sB = sG + C;
  stage_rows<TI, D, C>(sK, LD, k + ((long)start * Hg + hk) * D, (long)Hg * D, len);
  for (int t = threadIdx.x; t < C; t += kThreads) {
    const long gi = (long)h * Ttot + start + t;
    sG[t] = t < len ? g_t[gi] : 0.f;
    sB[t] = t < len ? load_beta(beta_t, beta_f32, gi) : 0.f;
  }
  __syncthreads();
  constexpr int NT = C / 16;
  const int w = wave_id(), l = lane_id();
  for (int tt = w; tt < NT * NT; tt += kWaves) {
    const int ti = tt / NT, tj = tt % NT;
    f32x4 acc = zero4();
    if (ti >= tj) mma_lds<TI>(acc, sK, LD, ti * 16, sK, LD, tj * 16, 0, D);
    const int j = tj * 16 + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = ti * 16 + 4 * (l >> 4) + e;
      if (i < len) {
        float val = 0.f;
        if (i > j) val = sB[i] * __expf(sG[i] - sG[j]) * acc[e];
        A[((long)(start + i) * H + h) * C + j] = val;
      }
    }
  }
}

// ------------------------------------------------------------------------- stage 4
template <typename TI> struct SolveType { typedef f16 type; };
template <> struct SolveType<float> { typedef float type; };

// Rows t < len of T (lower triangle of sM [C][ld]; the upper part written as zeros) to dst
// (row stride `stride` elements), eight elements per store.
template <typename TI, int C, typename TS>
__device__ __forceinline__ void store_T_rows(const TS* sM, int ld, TI* dst, long stride,
                                             int len) {
  constexpr int P8 = C / 8, OITER = (C * P8 + kThreads - 1) / kThreads;
#pragma unroll
  for (int it = 0; it < OITER; ++it) {
    const int i = threadIdx.x + it * kThreads;
    const int t = i / P8, j0 = (i - t * P8) * 8;
    if (i < C * P8 && t < len) {
      union {
        uint4 u[2];
        TI e[8];
      } o;
      union {
        uint4 u[sizeof(TS) / 2];
        TS e[8];
      } m;  // the row's 8 elements, one 16-byte LDS read per 16 bytes
#pragma unroll
      for (int q = 0; q < (int)sizeof(TS) / 2; ++q)
        m.u[q] = reinterpret_cast<const uint4*>(sM + t * ld + j0)[q];
#pragma unroll
      for (int e = 0; e < 8; ++e) o.e[e] = (TI)(j0 + e <= t ? (float)m.e[e] : 0.f);
      uint4* d = reinterpret_cast<uint4*>(dst + (long)t * stride + j0);
#pragma unroll
      for (int q = 0; q < (int)sizeof(TI) / 2; ++q) d[q] = o.u[q];
    }
  }
}

template <typename TI, int C>
__global__ __launch_bounds__(kThreads) void k_solve(const int32_t* table, const float* A,
                                                    TI* Tinv, int H) {
  const int4 ci = load_chunk(table, blockIdx.x);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y;
  typedef typename SolveType<TI>::type TS;
  constexpr int LD = C + pad_of<TS>();
  extern __shared__ __align__(16) char smem[];
  TS* sA = reinterpret_cast<TS*>(smem);
  TS* sM = sA + C * LD;
  float* sAd = reinterpret_cast<float*>(sM + C * LD);
  // A's rows in unrolled batches of eight 16-byte loads, all in flight together (rows past
  // the chunk's end read its last row and are zeroed at the store)
  constexpr int P4 = C / 4, ITER = C * P4 / kThreads, BATCH = ITER < 8 ? ITER : 8;
  static_assert(C * P4 % kThreads == 0 && ITER % BATCH == 0, "whole batches");
#pragma unroll
  for (int b0 = 0; b0 < ITER; b0 += BATCH) {
    f32x4 v[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int i = threadIdx.x + (b0 + q) * kThreads;
      const int t = i / P4, j0 = (i - t * P4) * 4;
      v[q] = *reinterpret_cast<const f32x4*>(A + ((long)(start + min(t, len - 1)) * H + h) * C + j0);
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int i = threadIdx.x + (b0 + q) * kThreads;
      const int t = i / P4, j0 = (i - t * P4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        const float x = t < len ? v[q][e] : 0.f;
        if ((t >> 4) == (j >> 4))
          sAd[(t >> 4) * 16 * kAdLd + (t & 15) * kAdLd + (j & 15)] = x;
        else
          sA[t * LD + j] = (TS)x;
      }
    }
  }
  __syncthreads();
  solve_tril<kWaves, C, TS>(sA, LD, sAd, sM, LD);
  store_T_rows<TI, C>(sM, LD, Tinv + ((long)start * H + h) * C, (long)H * C, len);
}

// The backward's stages 3 and 4 in one launch: A is built in LDS (the split of k_solve's
// staging: the diagonal blocks in fp32, the rest in the solve's type) and inverted there, so
// only T leaves the chip.  Same products and roundings as k_kkt followed by k_solve.
template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_kkt_solve(const int32_t* table, const TI* k,
                                                        const float* g_t, const void* beta_t,
                                                        int beta_f32, TI* Tinv, int Ttot,
                                                        int H, int Hg) {
  const int4 ci = load_chunk(table, blockIdx.x);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y, hk = h / (H / Hg);
  typedef typename SolveType<TI>::type TS;
  constexpr int LDK = D + pad_of<TI>(), LD = C + pad_of<TS>(), NT = C / 16;
  extern __shared__ __align__(16) char smem[];
  TS* sA = reinterpret_cast<TS*>(smem);
  TS* sM = sA + C * LD;
  float* sAd = reinterpret_cast<float*>(sM + C * LD);
  TI* sK = reinterpret_cast<TI*>(sAd + NT * 16 * kAdLd);
  float* sG = reinterpret_cast<float*>(sK + C * LDK);
  float* sB = sG + C;
  stage_rows<TI, D, C>(sK, LDK, k + ((long)start * Hg + hk) * D, (long)Hg * D, len);
  for (int t = threadIdx.x; t < C; t += kThreads) {
    const long gi = (long)h * Ttot + start + t;
    sG[t] = t < len ? g_t[gi] : 0.f;
    sB[t] = t < len ? load_beta(beta_t, beta_f32, gi) : 0.f;
  }
  __syncthreads();
  const int w = wave_id(), l = lane_id();
  for (int tt = w; tt < NT * NT; tt += kWaves) {
    const int ti = tt / NT, tj = tt % NT;
    f32x4 acc = zero4();
    if (ti >= tj) mma_lds<TI>(acc, sK, LDK, ti * 16, sK, LDK, tj * 16, 0, D);
    const int j = tj * 16 + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = ti * 16 + 4 * (l >> 4) + e;
      const float val = (i < len && i > j) ? sB[i] * __expf(sG[i] - sG[j]) * acc[e] : 0.f;
      if (ti == tj)
        sAd[ti * 16 * kAdLd + (i & 15) * kAdLd + (j & 15)] = val;
      else
        sA[i * LD + j] = (TS)val;
    }
  }
  __syncthreads();
  solve_tril<kWaves, C, TS>(sA, LD, sAd, sM, LD);
  store_T_rows<TI, C>(sM, LD, Tinv + ((long)start * H + h) * C, (long)H * C, len);
}

template <typename TI, int D, int C>
constexpr size_t kkt_solve_smem() {
  typedef typename SolveType<TI>::type TS;
  return 2 * C * (C + pad_of<TS>()) * sizeof(TS) + (C / 16) * 16 * kAdLd * 4 +
         C * (D + pad_of<TI>()) * sizeof(TI) + 2 * C * sizeof(float);
}

// ------------------------------------------------------------------------- stage 5
template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_wy(const int32_t* table, const TI* Tinv,
                                                 const TI* k, const TI* v, const float* g_t,
                                                 const void* beta_t, int beta_f32, TI* W,
                                                 TI* U, int Ttot, int H, int Hg) {
  const int4 ci = load_chunk(table, blockIdx.x);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y, hk = h / (H / Hg);
  constexpr int LD = C + pad_of<TI>();
  constexpr int PW = 64;  // output columns per panel
  constexpr int KS = Mma<TI>::KS;
  extern __shared__ __align__(16) char smem[];
  TI* sT = reinterpret_cast<TI*>(smem);
  TI* sP = sT + C * LD;
  float* sB = reinterpret_cast<float*>(sP + PW * LD);
  float* sEB = sB + C;
  stage_rows<TI, C, C>(sT, LD, Tinv + ((long)start * H + h) * C, (long)H * C, len);
  for (int t = threadIdx.x; t < C; t += kThreads) {
    const long gi = (long)h * Ttot + start + t;
    const float b = t < len ? load_beta(beta_t, beta_f32, gi) : 0.f;
    sB[t] = b;
    sEB[t] = t < len ? b * __expf(g_t[gi]) : 0.f;
  }
  const int w = wave_id(), l = lane_id();
  for (int pass = 0; pass < 2; ++pass) {
    const TI* src = pass ? k + ((long)start * Hg + hk) * D : v + ((long)start * H + h) * D;
    const long sstride = pass ? (long)Hg * D : (long)H * D;
    const float* scl = pass ? sEB : sB;
    TI* dst = pass ? W : U;
    for (int p0 = 0; p0 < D; p0 += PW) {
      __syncthreads();  // sB/sEB/sT written; previous panel consumed
      stage_rows_T<TI, PW, C>(sP, LD, src + p0, sstride, len, scl);
      __syncthreads();
      // wave w owns output columns [16w, 16w + 16) of the panel; T is lower-triangular,
      // so row block ti only needs k < 16 (ti + 1).
      for (int ti = 0; ti < C / 16; ++ti) {
        f32x4 acc = zero4();
        const int kend = ((ti + 1) * 16 + KS - 1) / KS * KS;
        mma_lds<TI>(acc, sT, LD, ti * 16, sP, LD, w * 16, 0, kend);
        const int col = p0 + w * 16 + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = ti * 16 + 4 * (l >> 4) + e;
          if (i < len) dst[((long)(start + i) * H + h) * D + col] = (TI)acc[e];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------- stage 6
// One workgroup per (sequence, head, 64-column slice).  Wave w owns state columns
// [16w, 16w+16) of the slice for all Dk rows, kept in accumulator tiles; W h and the
// K^T v_new update take the state / new values straight from registers.  Where each
// thread can hold one sub-block of the W, K and U tiles, the next chunk's tiles are loaded
// into registers while the current chunk is computed.
template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_h(const int32_t* table,
                                                      const int32_t* seq_chunks, const TI* k,
                                                      const TI* W, const TI* U,
                                                      const float* g_t, const float* h0,
                                                      TI* h_c, TI* v_new, float* ht, int Ttot,
                                                      int H, int Hg) {
  const int n = blockIdx.x, h = blockIdx.y, hk = h / (H / Hg);
  const int w = wave_id(), l = lane_id();
  const int scol = 16 * w + (l & 15);
  const int dv = blockIdx.z * 64 + scol;
  constexpr int NDK = D / 16, NT = C / 16;
  constexpr int LDW = D + pad_of<TI>(), LDK = C + pad_of<TI>(), LDU = 64 + pad_of<TI>();
  constexpr bool PRE = tile_copy_fits<TI, C, D, kThreads>() &&
                       tile_copy_fits<TI, C, 64, kThreads>();
  extern __shared__ __align__(16) char smem[];
  TI* sW = reinterpret_cast<TI*>(smem);
  TI* sKt = sW + C * LDW;
  TI* sU = sKt + D * LDK;  // [C][LDU], this slice of U (prefetching form only)
  float* sG = reinterpret_cast<float*>(sU + (PRE ? C * LDU : 0));

  f32x4 st[NDK];
  const long hoff = ((long)n * H + h) * D * D;
#pragma unroll
  for (int db = 0; db < NDK; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dk = 16 * db + 4 * (l >> 4) + e;
      st[db][e] = h0 ? h0[hoff + (long)dk * D + dv] : 0.f;
    }

  const int c0 = seq_chunks[n], c1 = seq_chunks[n + 1];
  // the prefetching form's register tiles (unused otherwise)
  struct Pre {
    TileCopy<TI, (PRE ? C : 64), (PRE ? D : 64), kThreads> w, k;
    TileCopy<TI, (PRE ? C : 64), 64, kThreads> u;
  };
  Pre pre;
  float gt = 0.f;
  int glen = 0;
  auto fetch = [&](int c) {
    const int4 ci = load_chunk(table, c);
    const int start = ci.y, len = ci.z;
    pre.w.load(W + ((long)start * H + h) * D, (long)H * D, len);
    pre.k.load(k + ((long)start * Hg + hk) * D, (long)Hg * D, len);
    pre.u.load(U + ((long)start * H + h) * D + blockIdx.z * 64, (long)H * D, len);
    gt = g_t[(long)h * Ttot + start + min((int)threadIdx.x, len - 1)];
    glen = len;
  };
  if constexpr (PRE) {
    if (c1 > c0) fetch(c0);
  }
  for (int c = c0; c < c1; ++c) {
    const int4 ci = load_chunk(table, c);
    const int start = ci.y, len = ci.z;
    const long coff = ((long)c * H + h) * D * D;
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h_c[coff + (long)(16 * db + 4 * (l >> 4) + e) * D + dv] = (TI)st[db][e];
    if constexpr (PRE) {
      pre.w.store_nat(sW, LDW);
      pre.k.store_trn(sKt, LDK);
      pre.u.store_nat(sU, LDU);
      if (threadIdx.x < C) sG[threadIdx.x] = (int)threadIdx.x < glen ? gt : 0.f;
      if (c + 1 < c1) fetch(c + 1);
    } else {
      stage_rows<TI, D, C>(sW, LDW, W + ((long)start * H + h) * D, (long)H * D, len);
      stage_rows_T<TI, D, C>(sKt, LDK, k + ((long)start * Hg + hk) * D, (long)Hg * D, len,
                             nullptr);
      for (int t = threadIdx.x; t < C; t += kThreads)
        sG[t] = t < len ? g_t[(long)h * Ttot + start + t] : 0.f;
    }
    __syncthreads();
    const float glast = sG[len - 1];
    f32x4 vn[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      f32x4 x = zero4();
      mma_accB<TI, NDK>(x, sW, LDW, tb * 16, 0, st, NDK);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + 4 * (l >> 4) + e;
        const long gi = ((long)(start + min(t, len - 1)) * H + h) * D + dv;
        const float u = PRE ? (float)sU[t * LDU + scol] : (float)U[gi];
        const float val = u - x[e];
        if (t < len) v_new[gi] = (TI)val;
        vn[tb][e] = t < len ? val * __expf(glast - sG[t]) : 0.f;
      }
    }
    const float eg = __expf(glast);
#pragma unroll
    for (int db = 0; db < NDK; ++db) {
      st[db] *= eg;
      mma_accB<TI, NT>(st[db], sKt, LDK, db * 16, 0, vn, NT);
    }
    __syncthreads();
  }
  if (ht) {
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ht[hoff + (long)(16 * db + 4 * (l >> 4) + e) * D + dv] = st[db][e];
  }
}

// ------------------------------------------------------------------------- stage 7
// One workgroup per (chunk, head).  P = (Q K^T * decay) is built once in LDS (K streamed
// in panels of at most 128 columns), then each 64-column panel of o is produced with
// Q h_c and P v_new taking h_c and v_new straight from registers (wave w owns 16 columns).
template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_o(const int32_t* table, const TI* q,
                                                      const TI* k, const TI* v_new,
                                                      const TI* h_c, const float* g_t, TI* o,
                                                      int Ttot, int H, int Hg, float scale) {
  const int c = blockIdx.x;
  const int4 ci = load_chunk(table, c);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y, hk = h / (H / Hg);
  const int w = wave_id(), l = lane_id();
  constexpr int KP = D < 128 ? D : 128;
  constexpr int NT = C / 16, NDK = D / 16;
  constexpr int LDQ = D + pad_of<TI>(), LDKP = KP + pad_of<TI>(), LDP = C + pad_of<TI>();
  constexpr int NLOW = NT * (NT + 1) / 2;
  constexpr int MAXT = (NLOW + kWaves - 1) / kWaves;
  extern __shared__ __align__(16) char smem[];
  TI* sQ = reinterpret_cast<TI*>(smem);
  TI* sK = sQ + C * LDQ;
  TI* sP = sK + C * LDKP;
  float* sG = reinterpret_cast<float*>(sP + C * LDP);

  stage_rows<TI, D, C>(sQ, LDQ, q + ((long)start * Hg + hk) * D, (long)Hg * D, len);
  for (int t = threadIdx.x; t < C; t += kThreads)
    sG[t] = t < len ? g_t[(long)h * Ttot + start + t] : 0.f;
  // (every lower tile of P is written below, and only those are read)

  // P^T tiles (rows j, columns i, i >= j) accumulate over K panels.
  f32x4 pacc[MAXT];
#pragma unroll
  for (int m = 0; m < MAXT; ++m) pacc[m] = zero4();
  for (int kp = 0; kp < D; kp += KP) {
    __syncthreads();
    stage_rows<TI, KP, C>(sK, LDKP, k + ((long)start * Hg + hk) * D + kp, (long)Hg * D, len);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXT; ++m) {
      const int u = w + kWaves * m;
      if (u < NLOW) {
        int ti = 0;
        while ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
        const int tj = u - ti * (ti + 1) / 2;
        mma_lds<TI>(pacc[m], sK, LDKP, tj * 16, sQ + kp, LDQ, ti * 16, 0, KP);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MAXT; ++m) {
    const int u = w + kWaves * m;
    if (u < NLOW) {
      int ti = 0;
      while ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
      const int tj = u - ti * (ti + 1) / 2;
      const int i = ti * 16 + (l & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = tj * 16 + 4 * (l >> 4) + e;
        const float val = (i >= j) ? __expf(sG[i] - sG[j]) * pacc[m][e] : 0.f;
        sP[i * LDP + j] = (TI)val;
      }
    }
  }
  __syncthreads();

  const long hcoff = ((long)c * H + h) * D * D;
#pragma unroll 1
  for (int p0 = 0; p0 < D; p0 += 64) {
    const int dv = p0 + 16 * w + (l & 15);
    // the Q h_c part of every row block first, so that h_c is dead before v_new is loaded
    // (both together do not fit in registers at D = 256)
    f32x4 acc[NT];
    {
      f32x4 hc[NDK];
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hc[db][e] = (float)h_c[hcoff + (long)(16 * db + 4 * (l >> 4) + e) * D + dv];
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        acc[tb] = zero4();
        mma_accB<TI, NDK>(acc[tb], sQ, LDQ, tb * 16, 0, hc, NDK);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tb][e] *= __expf(sG[tb * 16 + 4 * (l >> 4) + e]);
        sched_fence();  // one row block's fragments at a time (no spills at D = 256)
      }
    }
    f32x4 vt[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + 4 * (l >> 4) + e;
        const float x = (float)v_new[((long)(start + min(t, len - 1)) * H + h) * D + dv];
        vt[tb][e] = t < len ? x : 0.f;
      }
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      mma_accB<TI, NT>(acc[tb], sP, LDP, tb * 16, 0, vt, tb + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tb * 16 + 4 * (l >> 4) + e;
        if (t < len) o[((long)(start + t) * H + h) * D + dv] = (TI)(scale * acc[tb][e]);
      }
      sched_fence();
    }
  }
}

// The same stage with every operand staged in LDS by 16-byte loads issued together at the
// start (Q, K, h_c, v_new; v_new takes K's place once P is built) and the transposed
// operands of Q h_c and P v_new read from the natural tiles (frag_tr).  For the shapes whose
// tiles give every thread one sub-block and fit in LDS; wave w makes the row blocks w, w + 4,
// ... of o, all D columns.
template <typename TI, int D, int C>
constexpr bool chunk_o_tiled() {
  constexpr int LDQ = D + pad_of<TI>(), LDP = C + pad_of<TI>();
  return tile_copy_fits<TI, C, D, kThreads>() && tile_copy_fits<TI, D, D, kThreads>() &&
         (2 * C * LDQ + C * LDP + D * LDQ) * (int)sizeof(TI) + C * 4 <= 160 * 1024 &&
         C % 64 == 0 && D % 64 == 0;
}

template <typename TI, int D, int C>
constexpr size_t chunk_o_tiled_smem() {
  constexpr int LDQ = D + pad_of<TI>(), LDP = C + pad_of<TI>();
  return (size_t)(2 * C * LDQ + C * LDP + D * LDQ) * sizeof(TI) + C * sizeof(float);
}

template <typename TI, int D, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_o_tiled(const int32_t* table, const TI* q,
                                                            const TI* k, const TI* v_new,
                                                            const TI* h_c, const float* g_t,
                                                            TI* o, int Ttot, int H, int Hg,
                                                            float scale) {
  const int c = blockIdx.x;
  const int4 ci = load_chunk(table, c);
  const int start = ci.y, len = ci.z;
  if (len == 0) return;
  const int h = blockIdx.y, hk = h / (H / Hg);
  const int w = wave_id(), l = lane_id(), lg = l >> 4, lc = l & 15;
  typedef Mma<TI> MM;
  constexpr int NT = C / 16, NDK = D / 16, RPW = NT / kWaves;  // row blocks per wave
  constexpr int LDQ = D + pad_of<TI>(), LDP = C + pad_of<TI>();
  extern __shared__ __align__(16) char smem[];
  TI* sQ = reinterpret_cast<TI*>(smem);
  TI* sK = sQ + C * LDQ;  // K, then v_new
  TI* sV = sK;
  TI* sP = sK + C * LDQ;
  TI* sH = sP + C * LDP;
  float* sG = reinterpret_cast<float*>(sH + D * LDQ);

  TileCopy<TI, C, D, kThreads> bq, bk, bv;
  TileCopy<TI, D, D, kThreads> bh;
  const long qk0 = ((long)start * Hg + hk) * D, v0 = ((long)start * H + h) * D;
  bq.load(q + qk0, (long)Hg * D, len);
  bk.load(k + qk0, (long)Hg * D, len);
  bh.load(h_c + ((long)c * H + h) * D * D, D, D);
  bv.load(v_new + v0, (long)H * D, len);
  if (threadIdx.x < C) sG[threadIdx.x] = (int)threadIdx.x < len ? g_t[(long)h * Ttot + start + threadIdx.x] : 0.f;
  bq.store_nat(sQ, LDQ);
  bk.store_nat(sK, LDQ);
  bh.store_nat(sH, LDQ);
  // the tiles just above the diagonal of even block rows are read by the 32-deep P v
  // products and never written below: zero them
  for (int i = threadIdx.x; i < (NT / 2) * 16 * 2; i += kThreads) {
    const int p = i / 32, r = (i >> 1) & 15, half = i & 1;
    *reinterpret_cast<uint4*>(sP + (32 * p + r) * LDP + 32 * p + 16 + 8 * half) =
        make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // P[i][j] = (q_i . k_j) e^{Gc_i - Gc_j} for j <= i (lower tiles, dealt round robin)
  constexpr int NLOW = NT * (NT + 1) / 2, MAXT = (NLOW + kWaves - 1) / kWaves;
#pragma unroll
  for (int m = 0; m < MAXT; ++m) {
    const int u = w + kWaves * m;
    if (u < NLOW) {
      int ti = 0;
      while ((ti + 1) * (ti + 2) / 2 <= u) ++ti;
      const int tj = u - ti * (ti + 1) / 2;
      f32x4 acc = zero4();
      mma_lds<TI>(acc, sQ, LDQ, 16 * ti, sK, LDQ, 16 * tj, 0, D);
      const int j = 16 * tj + lc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * ti + 4 * lg + e;
        sP[i * LDP + j] = (TI)((i >= j) ? __expf(sG[i] - sG[j]) * acc[e] : 0.f);
      }
    }
  }
  __syncthreads();
  bv.store_nat(sV, LDQ);  // v_new where K was
  __syncthreads();

  // o = scale (diag(e^Gc) Q h_c + P v_new), row blocks w + 4 r of this wave
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int tb = w + kWaves * r;
    f32x4 acc[NDK];
#pragma unroll
    for (int cb = 0; cb < NDK; ++cb) acc[cb] = zero4();
    mma_steps<TI, D, 1, NDK>(
        [&](int, int kk) { return frag_ld<TI>(sQ, LDQ, 16 * tb, kk); },
        [&](int cb, int kk) { return frag_tr<TI>(sH, LDQ, 16 * cb, kk); },
        [&](auto& fa, auto& fb) {
#pragma unroll
          for (int cb = 0; cb < NDK; ++cb) acc[cb] = MM::mma(fa[0], fb[cb], acc[cb]);
        });
#pragma unroll
    for (int cb = 0; cb < NDK; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[cb][e] *= __expf(sG[16 * tb + 4 * lg + e]);
    const int kend = ((tb + 1) * 16 + MM::KS - 1) / MM::KS * MM::KS;
    for (int kk = 0; kk < kend; kk += MM::KS) {
      const auto fa = frag_ld<TI>(sP, LDP, 16 * tb, kk);
#pragma unroll
      for (int cb = 0; cb < NDK; ++cb)
        acc[cb] = MM::mma(fa, frag_tr<TI>(sV, LDQ, 16 * cb, kk), acc[cb]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * tb + 4 * lg + e;
      if (t < len) {
#pragma unroll
        for (int cb = 0; cb < NDK; ++cb)
          o[v0 + (long)t * H * D + 16 * cb + lc] = (TI)(scale * acc[cb][e]);
      }
    }
  }
}

// ------------------------------------------------------------------------- launchers
template <typename K>
hipError_t set_smem(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define GDN_TRY(x)                          \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

template <typename TI, int D, int C>
hipError_t run_staged(const Problem& p, const Stages& s, int stop_after, bool fuse34,
                      hipStream_t st) {
  const int MC = p.max_chunks;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  TI* Tinv = static_cast<TI*>(s.Tinv);
  TI* W = static_cast<TI*>(s.W);
  TI* U = static_cast<TI*>(s.U);
  TI* h_c = static_cast<TI*>(s.h_c);
  TI* v_new = static_cast<TI*>(s.v_new);
  const int bf = p.beta_f32 ? 1 : 0;

  k_chunk_table<<<1, 1024, 0, st>>>(p.cu, p.N, p.T, p.Ttot, C, MC, s.table, s.seq_chunks);
  GDN_TRY(hipGetLastError());
  if (MC == 0) return hipSuccess;

  k_cumsum<C><<<MC, kThreads, 0, st>>>(s.table, p.g, s.g_cum, p.H);
  GDN_TRY(hipGetLastError());
  if (stop_after == 1) return hipSuccess;

  if (p.Ttot > 0) {
    dim3 grid((p.Ttot + 63) / 64, (p.H + 63) / 64);
    k_transpose<float><<<grid, kThreads, 0, st>>>(s.g_cum, s.g_t, p.Ttot, p.H);
    GDN_TRY(hipGetLastError());
    if (p.beta_f32)
      k_transpose<float><<<grid, kThreads, 0, st>>>(static_cast<const float*>(p.beta),
                                                    static_cast<float*>(s.beta_t), p.Ttot, p.H);
    else
      k_transpose<uint16_t><<<grid, kThreads, 0, st>>>(static_cast<const uint16_t*>(p.beta),
                                                       static_cast<uint16_t*>(s.beta_t),
                                                       p.Ttot, p.H);
    GDN_TRY(hipGetLastError());
  }
  if (stop_after == 2) return hipSuccess;

  if (fuse34) {
    // the backward's shapes only (C = 64, D <= 128)
    if constexpr (C == 64 && D <= 128) {
      const size_t sm = kkt_solve_smem<TI, D, C>();
      GDN_TRY(set_smem(k_kkt_solve<TI, D, C>, sm));
      k_kkt_solve<TI, D, C><<<dim3(MC, p.H), kThreads, sm, st>>>(
          s.table, k, s.g_t, s.beta_t, bf, Tinv, p.Ttot, p.H, p.Hg);
      GDN_TRY(hipGetLastError());
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    const size_t sm = C * (D + pad_of<TI>()) * sizeof(TI) + 2 * C * sizeof(float);
    GDN_TRY(set_smem(k_kkt<TI, D, C>, sm));
    k_kkt<TI, D, C><<<dim3(MC, p.H), kThreads, sm, st>>>(s.table, k, s.g_t, s.beta_t, bf, s.A,
                                                         p.Ttot, p.H, p.Hg);
    GDN_TRY(hipGetLastError());
  }
  if (stop_after == 3) return hipSuccess;

  if (!fuse34) {
    typedef typename SolveType<TI>::type TS;
    const size_t sm = 2 * C * (C + pad_of<TS>()) * sizeof(TS) + (C / 16) * 16 * kAdLd * 4;
    GDN_TRY(set_smem(k_solve<TI, C>, sm));
    k_solve<TI, C><<<dim3(MC, p.H), kThreads, sm, st>>>(s.table, s.A, Tinv, p.H);
    GDN_TRY(hipGetLastError());
  }
  if (stop_after == 4) return hipSuccess;

  {
    const size_t sm = (C + 64) * (C + pad_of<TI>()) * sizeof(TI) + 2 * C * sizeof(float);
    GDN_TRY(set_smem(k_wy<TI, D, C>, sm));
    k_wy<TI, D, C><<<dim3(MC, p.H), kThreads, sm, st>>>(s.table, Tinv, k, v, s.g_t, s.beta_t,
                                                        bf, W, U, p.Ttot, p.H, p.Hg);
    GDN_TRY(hipGetLastError());
  }
  if (stop_after == 5) return hipSuccess;

  {
    constexpr bool pre = tile_copy_fits<TI, C, D, kThreads>() &&
                         tile_copy_fits<TI, C, 64, kThreads>();
    const size_t sm = (C * (D + pad_of<TI>()) + D * (C + pad_of<TI>()) +
                       (pre ? C * (64 + pad_of<TI>()) : 0)) * sizeof(TI) + C * sizeof(float);
    GDN_TRY(set_smem(k_chunk_h<TI, D, C>, sm));
    k_chunk_h<TI, D, C><<<dim3(p.N, p.H, D / 64), kThreads, sm, st>>>(
        s.table, s.seq_chunks, k, W, U, s.g_t, p.h0, h_c, v_new, stop_after ? nullptr : p.ht,
        p.Ttot, p.H, p.Hg);
    GDN_TRY(hipGetLastError());
  }
  if (stop_after == 6) return hipSuccess;

  if constexpr (chunk_o_tiled<TI, D, C>()) {
    const size_t sm = chunk_o_tiled_smem<TI, D, C>();
    GDN_TRY(set_smem(k_chunk_o_tiled<TI, D, C>, sm));
    k_chunk_o_tiled<TI, D, C><<<dim3(MC, p.H), kThreads, sm, st>>>(
        s.table, q, k, v_new, h_c, s.g_t, static_cast<TI*>(p.o), p.Ttot, p.H, p.Hg, p.scale);
    GDN_TRY(hipGetLastError());
  } else {
    constexpr int KP = D < 128 ? D : 128;
    const size_t sm = (C * (D + pad_of<TI>()) + C * (KP + pad_of<TI>()) +
                       C * (C + pad_of<TI>())) * sizeof(TI) + C * sizeof(float);
    GDN_TRY(set_smem(k_chunk_o<TI, D, C>, sm));
    k_chunk_o<TI, D, C><<<dim3(MC, p.H), kThreads, sm, st>>>(
        s.table, q, k, v_new, h_c, s.g_t, static_cast<TI*>(p.o), p.Ttot, p.H, p.Hg, p.scale);
    GDN_TRY(hipGetLastError());
  }
  return hipSuccess;
}

template <typename TI, int D>
hipError_t run_staged_c(const Problem& p, const Stages& s, int stop_after, bool fuse34,
                        hipStream_t st) {
  return p.C == 64 ? run_staged<TI, D, 64>(p, s, stop_after, fuse34, st)
                   : run_staged<TI, D, 128>(p, s, stop_after, fuse34, st);
}

template <typename TI>
hipError_t run_staged_d(const Problem& p, const Stages& s, int stop_after, bool fuse34,
                        hipStream_t st) {
  switch (p.D) {
    case 64: return run_staged_c<TI, 64>(p, s, stop_after, fuse34, st);
    case 128: return run_staged_c<TI, 128>(p, s, stop_after, fuse34, st);
    default: return run_staged_c<TI, 256>(p, s, stop_after, fuse34, st);
  }
}

}  // namespace

hipError_t launch_staged(const Problem& p, const Stages& s, int stop_after, hipStream_t st,
                         bool fuse_kkt_solve) {
  return p.f32 ? run_staged_d<float>(p, s, stop_after, fuse_kkt_solve, st)
               : run_staged_d<bf16>(p, s, stop_after, fuse_kkt_solve, st);
}

hipError_t launch_chunk_table(const Problem& p, const Stages& s, hipStream_t st) {
  k_chunk_table<<<1, 1024, 0, st>>>(p.cu, p.N, p.T, p.Ttot, p.C, p.max_chunks, s.table,
                                    s.seq_chunks);
  return hipGetLastError();
}

}  // namespace gdn
