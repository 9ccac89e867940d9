// Backward pass of the chunked gated delta rule (the FlashQLA how-to cites forward and
// backward speed-ups of the chunked operator; no page prints its formulas).  Written for
// gfx950 from the chunked forward's algebra.
//
// Per chunk (C = 64 tokens), with h the state at the chunk start (Dk x Dv), Gc the in-chunk
// prefix sum of g, gam_t = e^{Gc_t}, gC = gam at the chunk's last token, Gam_ij =
// e^{Gc_i - Gc_j}, T = (I + A)^-1 with A = strictly_lower(diag(beta) (K K^T * Gam)), and
//   R = diag(beta) (V - diag(gam) K h),   Delta = T R   (v_new),
//   O = scale (diag(gam) Q h + (Q K^T * Gam)_{i>=j} Delta),
//   h' = gC h + K^T diag(gC / gam) Delta,
// the gradients given dO and dh' (the gradient of the chunk-end state) are
//   dDelta = P^T dO + diag(gC / gam) K dh',        P = scale (Q K^T * Gam)_{i>=j}
//   dh     = gC dh' + scale Q^T diag(gam) dO - W^T dDelta,   W = T diag(beta gam) K
//   dR     = T^T dDelta,   dA = -(dR Delta^T)_{i>j},   dV = diag(beta) dR
//   dQ     = scale diag(gam) dO h^T + Mi K,            Mi = scale (dO Delta^T * Gam)_{i>=j}
//   dK     = Mi^T Q + (DB + DB^T) K + diag(gC / gam) Delta dh'^T - diag(beta gam) dR h^T,
//            DB = diag(beta) dA * Gam
//   dbeta  = rowsum(dR * (V - diag(gam) K h)) + rowsum(dA * K K^T * Gam)
//   dGc    = scale gam rowsum(dO * Q h) - (gC / gam) rowsum(Delta * K dh')
//            - beta gam rowsum(dR * K h) + rowsum(E) - colsum(E),
//            E = Mi * Q K^T + DB * K K^T,
//            and at the last token also sum_t (gC / gam_t) rowsum(Delta * K dh')_t
//            + gC <dh', h>;  dg = the in-chunk suffix sum of dGc.
//
// Two kernels follow the recomputation of the forward's chunk quantities (chunk table, Gc,
// T, the chunk-start states and v_new in the workspace):
//   k_bwd_dh     one workgroup per (sequence, head), a wave per 16 state columns (two per
//                wave, two workgroups per CU, on grids of many pairs): the chunks in
//                reverse, dh kept in accumulator tiles; writes dh' of every chunk, dR, and
//                dh0.  A packed batch's sequences run longest first.  Long sequences run it
//                per segment (twice: once from a zero end gradient for each segment's own
//                share, composed in reverse order across the segments, then from each
//                segment's true end gradient);
//   k_bwd_chunk  one resident workgroup per CU walking the (chunk, head) items: everything
//                else, in phases that stage their operands in LDS, with the next item's tiles
//                copied in while the current item's last products run.
// Value heads that share a q/k head run in one workgroup of the chunk kernel, which sums
// their dq and dk in registers in head order (no float atomics: the results do not depend
// on scheduling).
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_operands.h"

namespace gdn {

namespace {

// threads of the chunk workgroup: 8 waves, two 16-row blocks of the C x D outputs each.  The
// kernel also runs with 16 waves of one row block each (1024 threads; at D = 128 in bf16 it
// then holds 114 registers, four waves per SIMD), but the extra fragment reads made the
// headline backward slower (10.4 against 10.0 ms).
template <typename TI, int D>
constexpr int chunk_threads() { return 512; }

// Layout of the dh workgroup: each wave owns CB blocks of 16 state columns.  CB = 1: one
// wave per block, the tiles double-buffered by chunk parity (133 KB of LDS at D = 128, one
// workgroup per CU).  CB = 2 (bf16, D = 128, for grids of many (sequence, head) pairs): four
// waves of two blocks and single-buffered tiles copied straight into LDS (71 KB, two
// workgroups per CU, each one's barriers and loads hidden behind the other's work).
template <int CB>
constexpr bool dh_double() { return CB == 1; }
template <int D, int CB>
constexpr int dh_threads() { return 64 * D / (16 * CB); }
constexpr int kBC = 64;   // chunk length of the backward

__device__ __forceinline__ int4 chunk_of(const int32_t* table, int c) {
  return reinterpret_cast<const int4*>(table)[c];
}

template <typename TI, int ROWS, int COLS, int NTH>
using Blk = TileCopy<TI, ROWS, COLS, NTH>;

// A buffer resource over `bytes` bytes from base: a store whose per-lane offset lies past the
// end is dropped by the hardware (so rows past a chunk's end need no branch), and each
// store's address is a 32-bit offset into the resource (no per-store 64-bit arithmetic).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}

// One element of TI at byte offset voff + soff of the resource.
template <typename TI>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t rs, float x, int voff,
                                           int soff) {
  if constexpr (sizeof(TI) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (TI)x), rs, voff,
                                          soff, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), rs, voff, soff,
                                          0);
}

// Sum over the 16 lanes of a lane group (one accumulator row, its 16 columns), in the VALU by
// DPP (no LDS traffic): swaps within each quad of lanes, then the row rotated by 4 and by 8
// lanes.  Every lane ends with the row's sum, in an order that depends on the lane (callers
// take one lane's value).
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x124>(x);  // row_ror 4
  x += dpp_f<0x128>(x);  // row_ror 8
  return x;
}

// The elements of a row-major [.][ld] tile in the accumulator layout: lane l gets rows
// r0 + 4 (l / 16) + e, e = 0..3, of column c0 + l % 16.  bf16: one transposing read (its
// elements widened through 32-bit words); fp32: four reads.
template <typename TI>
__device__ __forceinline__ f32x4 acc_read(const TI* M, int ld, int r0, int c0, int lg,
                                          int lc) {
  f32x4 o;
  if constexpr (sizeof(TI) == 2) {
    const uint2 x = __builtin_bit_cast(uint2, read_tr4(M + (r0 + 4 * lg + (lc >> 2)) * ld + c0 +
                                                       4 * (lc & 3)));
    o[0] = __builtin_bit_cast(float, x.x << 16);
    o[1] = __builtin_bit_cast(float, x.x & 0xFFFF0000u);
    o[2] = __builtin_bit_cast(float, x.y << 16);
    o[3] = __builtin_bit_cast(float, x.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)M[(r0 + 4 * lg + e) * ld + c0 + lc];
  }
  return o;
}

// Four consecutive elements of TI from four floats (one 8- or 16-byte LDS store).
template <typename TI>
__device__ __forceinline__ void store4(TI* p, f32x4 v) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4*>(p) = o;
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

// Sum over the 4 lane groups (one accumulator column, 16 of its rows with the 4 elements).
__device__ __forceinline__ float sum4g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}


// One 16-byte copy per lane from global memory straight into LDS: lane l's 16 bytes land at
// lds + 16 l (lds is the same for the whole wave; M0 carries it, and the wait state the
// hardware needs between an M0 write and the copy that reads it is in the statement).  It is
// inline assembly because the compiler, when it issues such a copy itself, waits for it to
// land before every transposing LDS read that follows (it cannot tell those reads apart from
// the copy's target), which would serialise the copies with the products they are meant to
// overlap.  The compiler therefore does not know of the copy: the caller waits for it
// (wait_loads) before the barrier that publishes the tile, and touches nothing of the tile
// before then.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds) {
  const unsigned a = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(a) : "memory");
}

// Wave w's share (NW waves) of a direct HBM -> LDS copy of a ROWS x COLS tile of TI into the
// padded natural layout [ROWS][COLS + pad_of<TI>()]: rows of PR 16-byte pieces and one pad
// piece.  Each copy instruction writes 64 consecutive 16-byte LDS pieces, lane l the l-th, so
// piece p of the tile is row p / (PR + 1), piece p % (PR + 1); the pad piece re-reads its
// row's first piece.  Rows past len re-read row len - 1 (in bounds; every product masks those
// rows).  No registers hold the data: the copy lands in LDS on its own, and a wait for the
// wave's memory counter, then a barrier, make it visible to the workgroup.
template <typename TI, int ROWS, int COLS, int NW>
__device__ __forceinline__ void dma_tile(TI* dst, const TI* src, long stride, int len, int w,
                                         int l) {
  constexpr int VE = 16 / (int)sizeof(TI), PR = COLS / VE, PP = PR + 1;
  static_assert(COLS + pad_of<TI>() == PP * VE, "one pad piece per row");
  static_assert((ROWS * PP) % kWave == 0, "whole copy instructions");
  constexpr int NI = ROWS * PP / kWave;
#pragma unroll
  for (int j0 = 0; j0 < NI; j0 += NW) {
    const int j = j0 + w;
    if (j < NI) {
      const int p = kWave * j + l, r = p / PP, c = p % PP;
      lds_copy16(src + (long)min(r, len - 1) * stride + (c < PR ? c : 0) * VE,
                 dst + kWave * VE * j);
    }
  }
}

// Wait until this wave's loads (copies into LDS included) have landed.
__device__ __forceinline__ void wait_loads() {
  // s_waitcnt with vmcnt = 0 and expcnt, lgkmcnt at their maxima (no wait on those)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ------------------------------------------------------------------------- dh pass
// acc += M^T[col0 .. col0 + 15][k] * Bt[k][.] over k < 16 NKB, with M row-major [k][col] in
// LDS and Bt accumulator tiles whose rows run over k (the k order of mma_accB: 4 consecutive
// k per lane group and half).  bf16: M^T's fragments by transposing reads; fp32: strided
// reads.
template <typename TI, int NKB>
__device__ __forceinline__ void mma_accB_T(f32x4& acc, const TI* M, int ld, int col0,
                                           const f32x4* Bt) {
  const int l = lane_id(), c = l & 15, g = l >> 4;
  if constexpr (sizeof(TI) == 2) {
    static_assert(NKB % 2 == 0, "pairs of k blocks");
    const TI* p = M + (4 * g + (c >> 2)) * ld + col0 + 4 * (c & 3);
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2) {
      const bf16x4 a0 = read_tr4(p + 16 * kb * ld), a1 = read_tr4(p + (16 * kb + 16) * ld);
      const bf16x4 b0 = __builtin_convertvector(Bt[kb], bf16x4);
      const bf16x4 b1 = __builtin_convertvector(Bt[kb + 1], bf16x4);
      acc = Mma<bf16>::mma(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                           __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = Mma<TI>::mma(M[(16 * kb + 4 * g + i) * ld + col0 + c], Bt[kb][i], acc);
  }
}

// acc += A[arow0 .. + 15][k] * M[k][n0 .. n0 + 15] over k < K: A row-major in LDS (k
// contiguous), M row-major [k][n] in LDS, read by transposing reads (bf16) or strided reads.
template <typename TI, int K>
__device__ __forceinline__ void mma_lds_Bn(f32x4& acc, const TI* A, int lda, int arow0,
                                           const TI* M, int ldm, int n0) {
  const int l = lane_id(), c = l & 15, g = l >> 4;
  if constexpr (sizeof(TI) == 2) {
    const TI* pa = A + (arow0 + c) * lda + 4 * g;
    const TI* pm = M + (4 * g + (c >> 2)) * ldm + n0 + 4 * (c & 3);
#pragma unroll
    for (int k = 0; k < K; k += 32) {
      const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(pa + k);
      const bf16x4 a1 = *reinterpret_cast<const bf16x4*>(pa + k + 16);
      const bf16x4 b0 = read_tr4(pm + k * ldm), b1 = read_tr4(pm + (k + 16) * ldm);
      acc = Mma<bf16>::mma(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                           __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), acc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; k += 4)
      acc = Mma<TI>::mma(A[(arow0 + c) * lda + k + g], M[(k + g) * ldm + n0 + c], acc);
  }
}

// With W = T diag(beta gam) K, the update's W^T dDelta is K^T diag(beta gam) dR, dR = T^T
// dDelta: the pass reads rows of T (C x C) instead of W (C x D), and hands dR to the chunk
// kernel.  One workgroup per (sequence, head), wave w owning the state columns of blocks
// CB w .. CB w + CB - 1, so Q, K and T are read and P is built once per chunk.  Every tile
// sits in LDS in its natural layout (Q, K, dO [C][LDD]; T, P^T [C][LDC]); the transposed
// operands Q^T, K^T, T^T and dO^T are read from them directly.  Double-buffered (one tile set
// per chunk parity), storing the next chunk's tiles needs no barrier of its own.
template <typename TI, int D>
constexpr size_t dh_buf_bytes() {
  constexpr int LDD = D + pad_of<TI>(), LDC = kBC + pad_of<TI>();
  return (3 * kBC * LDD + kBC * LDC) * sizeof(TI) + 2 * kBC * sizeof(float);
}

template <typename TI, int D, int CB>
constexpr size_t dh_smem() {
  constexpr int LDC = kBC + pad_of<TI>();
  return (dh_double<CB>() ? 2 : 1) * dh_buf_bytes<TI, D>() + kBC * LDC * sizeof(TI);
}

template <typename TI, int D, int CB>
__global__ __launch_bounds__((dh_threads<D, CB>()), (dh_double<CB>() ? 1 : 2)) void k_bwd_dh(
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_chunks,
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ Tinv,
    const void* __restrict__ beta, int beta_f32, const TI* __restrict__ dO,
    const float* __restrict__ g_t, const float* __restrict__ dht, TI* __restrict__ dH,
    TI* __restrict__ dRo, float* __restrict__ dh0, const int32_t* __restrict__ order, int Ttot,
    int H, int Hg, float scale) {
  constexpr int C = kBC, NDK = D / 16, NT = C / 16, NW = D / (16 * CB);
  constexpr int NTH = dh_threads<D, CB>();
  constexpr bool DBUF = dh_double<CB>();
  constexpr int LDD = D + pad_of<TI>(), LDC = C + pad_of<TI>();
  // the run and head: with a longest-first order, workgroup rank (in launch order, heads
  // innermost) r takes run order[r / H], so the longest runs start first and the grid ends
  // with short ones; else run blockIdx.x, head blockIdx.y
  int n = blockIdx.x, h = blockIdx.y;
  if (order) {
    const int lin = (int)(blockIdx.x + blockIdx.y * gridDim.x);
    n = order[lin / H];
    h = lin % H;
  }
  const int hk = h / (H / Hg);
  const int w = wave_id(), l = lane_id();
  extern __shared__ __align__(16) char smem[];
  TI* sPt = reinterpret_cast<TI*>(smem + (DBUF ? 2 : 1) * dh_buf_bytes<TI, D>());  // P^T

  // dh tile (cb, db): rows (key index) 16 db + 4 (l/16) + e, column col(cb)
  auto col_of = [&](int cb) { return 16 * (CB * w + cb) + (l & 15); };
  f32x4 dh[CB][NDK];
  const long hoff = ((long)n * H + h) * D * D;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dh[cb][db][e] =
            dht ? dht[hoff + (long)(16 * db + 4 * (l >> 4) + e) * D + col_of(cb)] : 0.f;

  // Double-buffered: the chunk's operands are loaded one chunk ahead (into registers) while
  // the previous one is computed.  Single: they are copied straight into LDS at the chunk's
  // start (no registers held; the other workgroup on the CU runs meanwhile).
  const int c0 = seq_chunks[n], c1 = seq_chunks[n + 1];
  Blk<TI, C, D, NTH> bq, bk, bo;
  Blk<TI, C, C, NTH> bt;
  float gt = 0.f, bet = 0.f;
  int glen = 0;
  auto fetch_gates = [&](int start, int len) {
    const int tt = min((int)threadIdx.x, len - 1);
    gt = g_t[(long)h * Ttot + start + tt];
    bet = load_beta(beta, beta_f32, (long)(start + tt) * H + h);
    glen = len;
  };
  auto fetch = [&](int c) {
    const int4 ci = chunk_of(table, c);
    const int start = ci.y, len = ci.z;
    const long qk0 = ((long)start * Hg + hk) * D, v0 = ((long)start * H + h) * D;
    bq.load(q + qk0, (long)Hg * D, len);
    bk.load(k + qk0, (long)Hg * D, len);
    bt.load(Tinv + ((long)start * H + h) * C, (long)H * C, len);
    bo.load(dO + v0, (long)H * D, len);
    fetch_gates(start, len);
  };
  if constexpr (DBUF)
    if (c1 > c0) fetch(c1 - 1);
  for (int c = c1 - 1; c >= c0; --c) {
    const int4 ci = chunk_of(table, c);
    const int start = ci.y, len = ci.z;
    const long v0 = ((long)start * H + h) * D;
    // this chunk's buffer set: double-buffered, the other set was read by the previous
    // chunk, and the chunk before that, which read this one, finished before the previous
    // chunk's first barrier; single, every wave must be done with the previous chunk first
    if constexpr (!DBUF) __syncthreads();
    char* sb = smem + (DBUF ? ((c1 - 1 - c) & 1) * dh_buf_bytes<TI, D>() : 0);
    TI* sQ = reinterpret_cast<TI*>(sb);  // [C][LDD]
    TI* sK = sQ + C * LDD;               // [C][LDD]
    TI* sO = sK + C * LDD;               // [C][LDD]  dO
    TI* sT = sO + C * LDD;               // [C][LDC]  rows of T
    float* sG = reinterpret_cast<float*>(sT + C * LDC);
    float* sBeta = sG + C;
    if constexpr (DBUF) {
      bq.store_nat(sQ, LDD);
      bk.store_nat(sK, LDD);
      bt.store_nat(sT, LDC);
      bo.store_nat(sO, LDD);
    } else {
      // rows past len re-read row len - 1; every use masks them (P^T, dDelta, the update's
      // right-hand sides are zero there, T is zero above its diagonal)
      const long qk0 = ((long)start * Hg + hk) * D;
      dma_tile<TI, C, D, NW>(sQ, q + qk0, (long)Hg * D, len, w, l);
      dma_tile<TI, C, D, NW>(sK, k + qk0, (long)Hg * D, len, w, l);
      dma_tile<TI, C, C, NW>(sT, Tinv + ((long)start * H + h) * C, (long)H * C, len, w, l);
      dma_tile<TI, C, D, NW>(sO, dO + v0, (long)H * D, len, w, l);
      fetch_gates(start, len);
    }
    if (threadIdx.x < C) {
      const bool in = (int)threadIdx.x < glen;
      sG[threadIdx.x] = in ? gt : 0.f;
      sBeta[threadIdx.x] = in ? bet : 0.f;
    }
    if constexpr (DBUF) {
      if (c > c0) fetch(c - 1);
    } else {
      wait_loads();  // this wave's copies have landed
    }
    __syncthreads();
    // P^T: P[i][j] = scale (q_i . k_j) e^{Gc_i - Gc_j} for j <= i < len, stored at [j][i]
    // (wave w: tiles w, w + NW, ... of the 16)
#pragma unroll
    for (int m = 0; m < 16 / NW; ++m) {
      const int u = w + NW * m, ti = u >> 2, tj = u & 3;
      f32x4 acc = zero4();
      if (ti >= tj) mma_lds<TI>(acc, sQ, LDD, 16 * ti, sK, LDD, 16 * tj, 0, D);
      const int j = 16 * tj + (l & 15), i0 = 16 * ti + 4 * (l >> 4);
      const f32x4 gi = *reinterpret_cast<const f32x4*>(sG + i0);  // Gc of rows i0 .. i0 + 3
      const float gj = sG[j];
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        pv[e] = (i >= j && i < len) ? scale * acc[e] * __expf(gi[e] - gj) : 0.f;
      }
      store4<TI>(sPt + j * LDC + i0, pv);  // P^T row j, columns i0 .. i0 + 3
    }
    __syncthreads();
    const float gC = sG[len - 1], eC = __expf(gC);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = col_of(cb), cblk = 16 * (CB * w + cb);
      // dDelta (rows t, this lane's column) = P^T dO + (gC / gam_t) (K dh')
      f32x4 dd[NT];
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        f32x4 a = zero4(), x = zero4();
        mma_lds_Bn<TI, C>(a, sPt, LDC, 16 * tb, sO, LDD, cblk);
        mma_accB<TI, NDK>(x, sK, LDD, 16 * tb, 0, dh[cb], NDK);
        const f32x4 gt4 = *reinterpret_cast<const f32x4*>(sG + 16 * tb + 4 * (l >> 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tb + 4 * (l >> 4) + e;
          dd[tb][e] = t < len ? a[e] + __expf(gC - gt4[e]) * x[e] : 0.f;
        }
      }
      // dR = T^T dDelta
      f32x4 dr[NT];
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        dr[tb] = zero4();
        mma_accB_T<TI, NT>(dr[tb], sT, LDC, 16 * tb, dd);
      }
      // the chunk-end gradient dh' and dR, for the chunk-parallel kernel (not written by the
      // pass that only finds each segment's start gradient)
      if (dH) {
        constexpr int E = sizeof(TI);
        const auto rh = out_rsrc(dH + ((long)c * H + h) * D * D, D * D * E);
        const int hv = (4 * (l >> 4) * D + col) * E;
#pragma unroll
        for (int db = 0; db < NDK; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            store_elem<TI>(rh, dh[cb][db][e], hv, (16 * db + e) * D * E);
        // dR: the resource holds rows t < len; a store to a later row is dropped (its whole
        // offset is in the per-lane part, which the bounds check covers)
        const auto rr = out_rsrc(dRo + v0, (uint32_t)len * H * D * E);
        const int rstep = H * D * E;
#pragma unroll
        for (int tb = 0; tb < NT; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            store_elem<TI>(rr, dr[tb][e], (16 * tb + 4 * (l >> 4) + e) * rstep + col * E, 0);
      }
      // dh = gC dh' + scale Q^T diag(gam) dO - K^T diag(beta gam) dR
      f32x4 go[NT], nd[NT];
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        const int t0 = 16 * tb + 4 * (l >> 4);
        const f32x4 gt4 = *reinterpret_cast<const f32x4*>(sG + t0);
        const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sBeta + t0);
        const f32x4 o4 = acc_read(sO, LDD, 16 * tb, cblk, l >> 4, l & 15);  // dO[t][col]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + e;
          const float gam = t < len ? __expf(gt4[e]) : 0.f;
          go[tb][e] = scale * gam * o4[e];
          nd[tb][e] = -bt4[e] * gam * dr[tb][e];
        }
      }
#pragma unroll
      for (int db = 0; db < NDK; ++db) {
        dh[cb][db] *= eC;
        mma_accB_T<TI, NT>(dh[cb][db], sQ, LDD, 16 * db, go);
        mma_accB_T<TI, NT>(dh[cb][db], sK, LDD, 16 * db, nd);
      }
      // one column block at a time: its temporaries are dead before the next one's start
      if constexpr (CB > 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (dh0) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dh0[hoff + (long)(16 * db + 4 * (l >> 4) + e) * D + col_of(cb)] = dh[cb][db][e];
  }
}

// ------------------------------------------------------------------------- chunk gradients
// A TileCopy whose load takes the thread index as an argument: a loop that passes an index the
// compiler cannot see through recomputes the lane's addresses per call instead of holding
// them in registers across the loop.
template <typename TI, int ROWS, int COLS, int NTH>
struct TileRegs : TileCopy<TI, ROWS, COLS, NTH> {
  typedef TileCopy<TI, ROWS, COLS, NTH> B;
  __device__ __forceinline__ void load_at(const TI* src, long stride, int len_, int tid) {
    const int lo = tid & 63, hi = tid >> 6;
    const int bc = (lo & 7) + 8 * (hi % (B::BC / 8)), br = (lo >> 3) + 8 * (hi / (B::BC / 8));
    this->r0 = B::RB * br;
    this->c0 = B::V * bc;
    this->len = len_;
#pragma unroll
    for (int a = 0; a < B::RB; ++a)
      this->in[a].u = *reinterpret_cast<const uint4*>(
          src + (long)min(this->r0 + a, len_ - 1) * stride + this->c0);
  }
};


// One workgroup of 4 RW waves per resident slot; it walks the (chunk, head) items b, b + G,
// b + 2 G, ... (G workgroups, items with tokens only; RW = 2 or 4 row groups, RPW = 4 / RW).
// Wave w = 4 rh + cw: in the C x D products it owns the row blocks RPW rh .. RPW rh + RPW - 1
// and the column blocks cw + 4 m (m < D / 64); in the C x C products the row block cw and
// the column blocks RPW rh .. RPW rh + RPW - 1.  Every tile sits in LDS in its natural
// layout and the transposed operands are read from it (frag_tr), so h and dh' are each
// loaded once and every product that needs them runs while they are resident.  While one
// item's last products run, the next item's h, dR, dO and Delta are copied into the LDS
// tiles those products no longer read, and its K, Q and V load into registers.
template <typename TI, int D>
struct ChunkLds {
  static constexpr int C = kBC;
  static constexpr int LDD = D + pad_of<TI>(), LDC = C + pad_of<TI>();
  static constexpr int P = C * LDD;   // a C x D panel
  static constexpr int BIG = D * LDD; // a D x D matrix
  static constexpr int CC = C * LDC;  // a C x C matrix
  static_assert(P <= 2 * CC, "V fits in the two C x C tiles");
  static constexpr size_t bytes = (5 * P + BIG + 2 * CC) * sizeof(TI) + 26 * C * sizeof(float);
};

template <typename TI, int D, bool GRP>
__global__ __launch_bounds__((chunk_threads<TI, D>())) void k_bwd_chunk(
    const int32_t* __restrict__ table, int n_chunks, const TI* __restrict__ q,
    const TI* __restrict__ k, const TI* __restrict__ v, const void* __restrict__ beta,
    int beta_f32, const float* __restrict__ g_t, const TI* __restrict__ h_c,
    const TI* __restrict__ v_new, const TI* __restrict__ dR, const TI* __restrict__ dH,
    const TI* __restrict__ dO, void* __restrict__ dq, void* __restrict__ dk,
    void* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta, int qk_rows,
    int gsz, int Ttot, int H, int Hg, float scale, int grad_bf16) {
  typedef ChunkLds<TI, D> L;
  typedef Mma<TI> MM;
  constexpr int C = kBC, CBW = D / 64, N2 = chunk_threads<TI, D>();  // CBW: column blocks
                                                                      // per wave
  constexpr int NW = N2 / kWave;
  constexpr int RW = N2 / 256, RPW = 4 / RW;  // row groups of waves; row blocks per wave
  constexpr int LDD = L::LDD, LDC = L::LDC;
  constexpr int VE = 16 / (int)sizeof(TI), PR = D / VE;  // 16-byte pieces of a D row
  // GRP = false: an item is (chunk, value head); GRP: (chunk, q/k head), whose gsz value heads
  // run one after another on the resident K and Q, their dq and dk summed in registers (in
  // head order: deterministic)
  const int Hy = GRP ? Hg : H;
  const int n_items = n_chunks * Hy;
  const int nr = GRP ? gsz : 1;
  extern __shared__ __align__(16) char smem[];
  TI* sK = reinterpret_cast<TI*>(smem);
  TI* sQ = sK + L::P;
  TI* sC = sQ + L::P;            // dR
  TI* sO = sC + L::P;            // dO
  TI* sDl = sO + L::P;           // Delta
  TI* sBig = sDl + L::P;         // h, then dh'
  // Mi and DB are stored transposed (four elements per store) unless heads are grouped, where
  // the four values held for those stores cost registers the grouped loop does not have
  constexpr bool MT = !GRP;
  TI* sMi = sBig + L::BIG;       // V ([C][LDD] over both C x C tiles) in phase B, then Mi
  TI* sDB = sMi + L::CC;         // DB
  TI* sV = sMi;
  float* sG = reinterpret_cast<float*>(sDB + L::CC);
  float* sBeta = sG + C;
  // sPart [16 C]: the row dots' parts [quantity x][column wave][C] (x = 0..3); after they
  // are summed: rowsum(E) per row group of waves at 8 C, rowsum(dA * KK * Gam) per row
  // group at 12 C (at most four groups each)
  float* sPart = sBeta + C;
  float* sRD = sPart + 16 * C;   // [4][C] the row dots (1: Delta.K dh', 2: dR.K h, 3: dR.V);
                                 // its first C floats hold the parts of <dh', h>
  float* sColE = sRD + 4 * C;    // [4 row blocks][C] partial colsum(E)
  float* sHdh = sRD;              // one part per wave (at most C waves)
  float* sRowE = sPart + 8 * C;
  float* sRowB = sPart + 12 * C;

  // the next item at or after i (stride: the grid) that has tokens; n_items if none
  auto next_item = [&](int i) {
    while (i < n_items && chunk_of(table, i / Hy).z == 0) i += (int)gridDim.x;
    return i < n_items ? i : n_items;
  };
  // the value head of unit r of item i, and the offsets of its token rows and h_c / dh'
  auto value_head = [&](int i, int r) { return GRP ? (i % Hy) * gsz + r : i % Hy; };
  // copies of a unit's h (part 0) or its dR, dO and Delta (part 1) into LDS (the tiles must be
  // free)
  auto copy_unit = [&](int i, int r, int part) {
    const int cc = i / Hy, hv = value_head(i, r);
    const int4 ti = chunk_of(table, cc);
    int t = threadIdx.x;
    opaque(t);
    const int w = t >> 6, l = t & 63;
    if (part == 0) {
      dma_tile<TI, D, D, NW>(sBig, h_c + ((long)cc * H + hv) * D * D, D, D, w, l);
    } else {
      const long tv = ((long)ti.y * H + hv) * D;
      dma_tile<TI, C, D, NW>(sC, dR + tv, (long)H * D, ti.z, w, l);
      dma_tile<TI, C, D, NW>(sO, dO + tv, (long)H * D, ti.z, w, l);
      dma_tile<TI, C, D, NW>(sDl, v_new + tv, (long)H * D, ti.z, w, l);
    }
  };
  // K and Q (when the unit starts an item or heads are not grouped) and V of a unit, into
  // registers
  TileRegs<TI, C, D, N2> bk, bq, bv;
  auto load_unit = [&](int i, int r) {
    const int4 ti = chunk_of(table, i / Hy);
    const int hk = GRP ? i % Hy : (i % Hy) / (H / Hg);
    int t = threadIdx.x;
    opaque(t);
    if (!GRP || r == 0) {
      const long o = ((long)ti.y * Hg + hk) * D;
      bk.load_at(k + o, (long)Hg * D, ti.z, t);
      bq.load_at(q + o, (long)Hg * D, ti.z, t);
    }
    bv.load_at(v + ((long)ti.y * H + value_head(i, r)) * D, (long)H * D, ti.z, t);
  };

  int it = next_item((int)blockIdx.x);
  if (it >= n_items) return;
  copy_unit(it, 0, 0);
  copy_unit(it, 0, 1);
  load_unit(it, 0);
#pragma unroll 1
  for (;;) {
  const int c = it / Hy;
  const int4 ci = chunk_of(table, c);
  const int start = ci.y, len = ci.z;
  const int hk = GRP ? it % Hy : (it % Hy) / (H / Hg);
  const int hq = GRP ? hk : (qk_rows == H ? it % Hy : hk);  // dq, dk row
  const int next_it = next_item(it + (int)gridDim.x);
  f32x4 aq[RPW][CBW], ak[RPW][CBW];  // dq and dk, summed over the value heads
#pragma unroll
  for (int b = 0; b < RPW; ++b)
#pragma unroll
    for (int m = 0; m < CBW; ++m) aq[b][m] = ak[b][m] = zero4();
#pragma unroll 1
  for (int r = 0; r < nr; ++r) {
  // lane and wave indices re-derived per unit, so that the fragment addresses built from
  // them are not hoisted out of the loops and kept live across them
  int tid = threadIdx.x;
  opaque(tid);
  const int w = tid >> 6, l = tid & 63, lg = l >> 4, lc = l & 15;
  const int cw = w & 3, rh = w >> 2;
  const int h = value_head(it, r);
  // the next unit: the next value head of this item, or the next item's first
  const int nit = r + 1 < nr ? it : next_it, nrr = r + 1 < nr ? r + 1 : 0;
  const long v0 = ((long)start * H + h) * D;
  const long hcoff = ((long)c * H + h) * D * D;
  // the previous unit is done with the LDS, and this unit's copies have landed
  wait_loads();
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    sG[t] = t < len ? g_t[(long)h * Ttot + start + t] : 0.f;
    sBeta[t] = t < len ? load_beta(beta, beta_f32, (long)(start + t) * H + h) : 0.f;
  }
  if (!GRP || r == 0) {
    bk.store_nat(sK, LDD);
    bq.store_nat(sQ, LDD);
  }
  bv.store_nat(sV, LDD);
  Blk<TI, D, D, N2> bd;
  bd.load(dH + hcoff, D, D);  // dh', stored once h is no longer read
  __syncthreads();  // Gc, beta, K, Q, V
  // dV = diag(beta) dR, from the copied dR (fp32, or rounded once to bf16)
  for (int i = tid; i < C * PR; i += N2) {
    const int t = i / PR, pc = i % PR;
    if (t < len) {
      typename Blk<TI, C, D, N2>::Vec x;
      x.u = *reinterpret_cast<const uint4*>(sC + t * LDD + pc * VE);
      const float bt = sBeta[t];
      const long di = v0 + (long)t * H * D + pc * VE;
      bool done = false;
      if constexpr (sizeof(TI) == 2) {  // bf16 gradients come with bf16 inputs only
        if (grad_bf16) {
          typename Blk<bf16, C, D, N2>::Vec o;
#pragma unroll
          for (int e = 0; e < VE; ++e) o.e[e] = (bf16)(bt * (float)x.e[e]);
          *reinterpret_cast<uint4*>(static_cast<bf16*>(dv) + di) = o.u;
          done = true;
        }
      }
      if (!done) {
        float* dst = static_cast<float*>(dv) + di;
#pragma unroll
        for (int q4 = 0; q4 < VE / 4; ++q4) {
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = bt * (float)x.e[4 * q4 + e];
          *reinterpret_cast<f32x4*>(dst + 4 * q4) = o;
        }
      }
    }
  }

  // fragment readers of the C x D products: rows 32 rh + 16 i of a [C][LD] panel; the
  // B operands of columns 16 (cw + 4 j): natural rows of a [.][LD] matrix, or M^T from M
  auto rows = [&](const TI* Pm, int ld) {
    return [=](int i, int kk) { return frag_ld<TI>(Pm, ld, 16 * RPW * rh + 16 * i, kk); };
  };
  auto cols = [&](const TI* Pm, int ld) {
    return [=](int j, int kk) { return frag_ld<TI>(Pm, ld, 16 * (cw + 4 * j), kk); };
  };
  auto colsT = [&](const TI* Pm, int ld) {
    return [=](int j, int kk) { return frag_tr<TI>(Pm, ld, 16 * (cw + 4 * j), kk); };
  };

  // ---- phase B, h resident: K h, dO h^T (into aq), dR h^T (into ak), row dots.  aq and ak
  // carry dq and dk summed over the value heads of the item
  {
    f32x4 Kh[RPW][CBW], tq[RPW][CBW], tk[RPW][CBW];
#pragma unroll
    for (int b = 0; b < RPW; ++b)
#pragma unroll
      for (int m = 0; m < CBW; ++m) Kh[b][m] = tq[b][m] = tk[b][m] = zero4();
    mma_steps<TI, D, RPW, CBW>(rows(sK, LDD), colsT(sBig, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
      for (int b = 0; b < RPW; ++b)
#pragma unroll
        for (int m = 0; m < CBW; ++m) Kh[b][m] = MM::mma(fa[b], fb[m], Kh[b][m]);
    });
    mma_steps<TI, D, 2 * RPW, CBW>(
        [&](int i, int kk) {
          return frag_ld<TI>(i < RPW ? sO : sC, LDD, 16 * RPW * rh + 16 * (i % RPW), kk);
        },
        cols(sBig, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
          for (int b = 0; b < RPW; ++b)
#pragma unroll
            for (int m = 0; m < CBW; ++m) {
              tq[b][m] = MM::mma(fa[b], fb[m], tq[b][m]);
              tk[b][m] = MM::mma(fa[RPW + b], fb[m], tk[b][m]);
            }
        });
    // row dots over the wave's columns: dR.K h, dR.V, Q.(dO h^T) = dO.Q h
#pragma unroll
    for (int b = 0; b < RPW; ++b) {
      f32x4 eC[CBW], eV[CBW], eQ[CBW];  // dR, V and Q in the accumulator layout
#pragma unroll
      for (int m = 0; m < CBW; ++m) {
        const int r0 = 16 * (RPW * rh + b), c0 = 16 * (cw + 4 * m);
        eC[m] = acc_read(sC, LDD, r0, c0, lg, lc);
        eV[m] = acc_read(sV, LDD, r0, c0, lg, lc);
        eQ[m] = acc_read(sQ, LDD, r0, c0, lg, lc);
      }
      // Gc and beta of the lane's four rows
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(sG + 16 * (RPW * rh + b) + 4 * lg);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * (RPW * rh + b) + 4 * lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * (RPW * rh + b) + 4 * lg + e;
        float p0 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int m = 0; m < CBW; ++m) {
          const float r = eC[m][e];
          p2 += r * Kh[b][m][e];
          p3 += r * eV[m][e];
          p0 += eQ[m][e] * tq[b][m][e];
        }
        p0 = sum16(p0);
        p2 = sum16(p2);
        p3 = sum16(p3);
        if (lc == 0) {
          sPart[cw * C + t] = p0;
          sPart[(8 + cw) * C + t] = p2;
          sPart[(12 + cw) * C + t] = p3;
        }
        const float gam = __expf(g4[e]);
#pragma unroll
        for (int m = 0; m < CBW; ++m) {
          aq[b][m][e] += scale * gam * tq[b][m][e];
          ak[b][m][e] -= b4[e] * gam * tk[b][m][e];
        }
      }
    }
  }
  {
    // <dh', h> from the held dh' blocks and the resident h (parts per wave, in order)
    const float part = sum4g(sum16(bd.dot_nat(sBig, LDD)));
    if (l == 0) sHdh[w] = part;
  }
  __syncthreads();
  bd.store_nat(sBig, LDD);  // dh'
  __syncthreads();

  // ---- phase B', dh' resident: K dh' (row dot with Delta) and Delta dh'^T (into ak)
  const float gC = sG[len - 1];
  {
    f32x4 Kd[RPW][CBW], X[RPW][CBW];
#pragma unroll
    for (int b = 0; b < RPW; ++b)
#pragma unroll
      for (int m = 0; m < CBW; ++m) Kd[b][m] = X[b][m] = zero4();
    mma_steps<TI, D, RPW, CBW>(rows(sK, LDD), colsT(sBig, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
      for (int b = 0; b < RPW; ++b)
#pragma unroll
        for (int m = 0; m < CBW; ++m) Kd[b][m] = MM::mma(fa[b], fb[m], Kd[b][m]);
    });
    mma_steps<TI, D, RPW, CBW>(rows(sDl, LDD), cols(sBig, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
      for (int b = 0; b < RPW; ++b)
#pragma unroll
        for (int m = 0; m < CBW; ++m) X[b][m] = MM::mma(fa[b], fb[m], X[b][m]);
    });
#pragma unroll
    for (int b = 0; b < RPW; ++b) {
      f32x4 eD[CBW];  // Delta in the accumulator layout
#pragma unroll
      for (int m = 0; m < CBW; ++m)
        eD[m] = acc_read(sDl, LDD, 16 * (RPW * rh + b), 16 * (cw + 4 * m), lg, lc);
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(sG + 16 * (RPW * rh + b) + 4 * lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * (RPW * rh + b) + 4 * lg + e;
        float p1 = 0.f;
        const float r = __expf(gC - g4[e]);
#pragma unroll
        for (int m = 0; m < CBW; ++m) {
          p1 += eD[m][e] * Kd[b][m][e];
          ak[b][m][e] += r * X[b][m][e];
        }
        p1 = sum16(p1);
        if (lc == 0) sPart[(4 + cw) * C + t] = p1;
      }
    }
  }
  __syncthreads();  // row-dot parts complete; V and dh' read for the last time
  // dh' is read no more in this unit: copy the next unit's h into its tile
  if (nit < n_items) copy_unit(nit, nrr, 0);
  if (tid < 3 * C) {
    const int x = 1 + tid / C, t = tid % C;
    sRD[x * C + t] = sPart[(4 * x) * C + t] + sPart[(4 * x + 1) * C + t] +
                     sPart[(4 * x + 2) * C + t] + sPart[(4 * x + 3) * C + t];
  }

  // ---- phase C: the C x C products and their elementwise terms
  f32x4 KK[RPW], QK[RPW], E1[RPW], RD[RPW];
#pragma unroll
  for (int b = 0; b < RPW; ++b) KK[b] = QK[b] = E1[b] = RD[b] = zero4();
  mma_steps<TI, D, 2, RPW>(
      [&](int i, int kk) { return frag_ld<TI>(i ? sQ : sK, LDD, 16 * cw, kk); },
      [&](int j, int kk) { return frag_ld<TI>(sK, LDD, 16 * RPW * rh + 16 * j, kk); },
      [&](auto& fa, auto& fb) {
#pragma unroll
        for (int b = 0; b < RPW; ++b) {
          KK[b] = MM::mma(fa[0], fb[b], KK[b]);
          QK[b] = MM::mma(fa[1], fb[b], QK[b]);
        }
      });
  mma_steps<TI, D, 2, RPW>(
      [&](int i, int kk) { return frag_ld<TI>(i ? sC : sO, LDD, 16 * cw, kk); },
      [&](int j, int kk) { return frag_ld<TI>(sDl, LDD, 16 * RPW * rh + 16 * j, kk); },
      [&](auto& fa, auto& fb) {
#pragma unroll
        for (int b = 0; b < RPW; ++b) {
          E1[b] = MM::mma(fa[0], fb[b], E1[b]);
          RD[b] = MM::mma(fa[1], fb[b], RD[b]);
        }
      });
  __syncthreads();  // the row-dot parts are summed before sRowE / sRowB reuse their space
  // dR, dO and Delta are read no more in this unit: copy the next unit's into their tiles
  if (nit < n_items) copy_unit(nit, nrr, 1);
  float rowE[4] = {0.f, 0.f, 0.f, 0.f}, rowB[4] = {0.f, 0.f, 0.f, 0.f};
  // Gc and beta of the lane's four rows i
  const f32x4 gi4 = *reinterpret_cast<const f32x4*>(sG + 16 * cw + 4 * lg);
  const f32x4 bi4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * cw + 4 * lg);
#pragma unroll
  for (int b = 0; b < RPW; ++b) {
    const int j = 16 * (RPW * rh + b) + lc;
    const float gj = sG[j];
    float colE = 0.f;
    f32x4 mi4, db4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * cw + 4 * lg + e;
      const bool in = i < len && j < len;
      const float gam = (in && i >= j) ? __expf(gi4[e] - gj) : 0.f;
      const float mi = (i >= j) ? scale * E1[b][e] * gam : 0.f;
      const float da = (in && i > j) ? -RD[b][e] : 0.f;
      const float db = bi4[e] * da * gam;
      const float ee = mi * QK[b][e] + db * KK[b][e];
      rowE[e] += ee;
      rowB[e] += da * KK[b][e] * gam;
      colE += ee;
      if constexpr (MT) {
        mi4[e] = mi;
        db4[e] = db;
      } else {
        sMi[i * LDC + j] = (TI)mi;
        sDB[i * LDC + j] = (TI)db;
      }
    }
    if constexpr (MT) {
      // stored transposed: the lane's four rows i are consecutive there
      store4<TI>(sMi + j * LDC + 16 * cw + 4 * lg, mi4);
      store4<TI>(sDB + j * LDC + 16 * cw + 4 * lg, db4);
    }
    colE = sum4g(colE);
    if (lg == 0) sColE[cw * C + j] = colE;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float re = sum16(rowE[e]), rb = sum16(rowB[e]);
    if (lc == 0) {
      sRowE[rh * C + 16 * cw + 4 * lg + e] = re;
      sRowB[rh * C + 16 * cw + 4 * lg + e] = rb;
    }
  }
  __syncthreads();

  // ---- phase D: Mi K into aq; (DB + DB^T) K and Mi^T Q into ak.  Fragments of a matrix
  // held as stored are natural reads, of its transpose transposing reads
  auto frag_m = [&](const TI* Pm, int r0, int kk, bool transposed) {
    return transposed == MT ? frag_ld<TI>(Pm, LDC, r0, kk) : frag_tr<TI>(Pm, LDC, r0, kk);
  };
  mma_steps<TI, C, 2 * RPW, CBW>(
      [&](int i, int kk) {
        const TI* Pm = i >= RPW ? sDB : sMi;
        return frag_m(Pm, 16 * RPW * rh + 16 * (i % RPW), kk, false);
      },
      colsT(sK, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
        for (int b = 0; b < RPW; ++b)
#pragma unroll
          for (int m = 0; m < CBW; ++m) {
            aq[b][m] = MM::mma(fa[b], fb[m], aq[b][m]);
            ak[b][m] = MM::mma(fa[RPW + b], fb[m], ak[b][m]);
          }
      });
  mma_steps<TI, C, RPW, CBW>(
      [&](int i, int kk) { return frag_m(sDB, 16 * RPW * rh + 16 * i, kk, true); },  // DB^T
      colsT(sK, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
        for (int b = 0; b < RPW; ++b)
#pragma unroll
          for (int m = 0; m < CBW; ++m) ak[b][m] = MM::mma(fa[b], fb[m], ak[b][m]);
      });
  mma_steps<TI, C, RPW, CBW>(
      [&](int i, int kk) { return frag_m(sMi, 16 * RPW * rh + 16 * i, kk, true); },  // Mi^T
      colsT(sQ, LDD), [&](auto& fa, auto& fb) {
#pragma unroll
        for (int b = 0; b < RPW; ++b)
#pragma unroll
          for (int m = 0; m < CBW; ++m) ak[b][m] = MM::mma(fa[b], fb[m], ak[b][m]);
      });
  // the next unit's K, Q and V into registers (stored once every wave is past phase D)
  if (nit < n_items) load_unit(nit, nrr);

  // ---- dbeta and dg: wave 0, lane t = token t (C = 64 = one wave).  dg is the suffix sum of
  // dGc in the chunk; the last token's dGc also takes sum_t (gC / gam_t) rowsum(Delta * K
  // dh')_t + gC <dh', h>.  Butterfly sums and a wave scan: a fixed order (deterministic).
  static_assert(C == kWave, "one token per lane of wave 0");
  if (w == 0) {
    const int t = l;
    float dgc = 0.f, db = 0.f, share = 0.f;
    if (t < len) {
      const float gam = __expf(sG[t]), r = __expf(gC - sG[t]);
      const float colE = sColE[t] + sColE[C + t] + sColE[2 * C + t] + sColE[3 * C + t];
      const float rq = sPart[t] + sPart[C + t] + sPart[2 * C + t] + sPart[3 * C + t];
      float rowB = 0.f, rowE = 0.f;
#pragma unroll
      for (int x = 0; x < RW; ++x) {
        rowB += sRowB[x * C + t];
        rowE += sRowE[x * C + t];
      }
      db = sRD[3 * C + t] - gam * sRD[2 * C + t] + rowB;
      dgc = scale * gam * rq - r * sRD[C + t] - sBeta[t] * gam * sRD[2 * C + t] + rowE - colE;
      share = r * sRD[C + t];  // the last token's share of h' = gC h + ...
      dbeta[(long)(start + t) * H + h] = db;
    }
    const float hdh = t < N2 / 64 ? sHdh[t] : 0.f;
    const float tot = sum4g(sum16(share)) + __expf(gC) * sum4g(sum16(hdh));
    if (t == len - 1) dgc += tot;
    // suffix sums: lane u scans token C - 1 - u, then each token takes its own
    const float sc = wave_incl_scan(__shfl(dgc, C - 1 - t, kWave));
    const float suf = __shfl(sc, C - 1 - t, kWave);
    if (t < len) dg[(long)(start + t) * H + h] = suf;
  }
  }
  {
    const int w = wave_id(), l = lane_id(), lg = l >> 4, lc = l & 15;
    const int cw = w & 3, rh = w >> 2;
    const long dq0 = ((long)start * qk_rows + hq) * D;
#pragma unroll
    for (int b = 0; b < RPW; ++b)
#pragma unroll
      for (int m = 0; m < CBW; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * (RPW * rh + b) + 4 * lg + e;
          if (t < len) {
            const long gi = dq0 + (long)t * qk_rows * D + 16 * (cw + 4 * m) + lc;
            if (grad_bf16) {
              static_cast<bf16*>(dq)[gi] = (bf16)aq[b][m][e];
              static_cast<bf16*>(dk)[gi] = (bf16)ak[b][m][e];
            } else {
              static_cast<float*>(dq)[gi] = aq[b][m][e];
              static_cast<float*>(dk)[gi] = ak[b][m][e];
            }
          }
        }
  }
  it = next_it;
  if (it >= n_items) break;
  }
}

template <typename F>
hipError_t set_lds(F f, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define GDN_BTRY(x)                     \
  do {                                  \
    hipError_t e_ = (x);                \
    if (e_ != hipSuccess) return e_;    \
  } while (0)

template <typename TI, int D, int CB>
hipError_t run_bwd_dh_cb(const Problem& p, const BwdBuffers& b, int runs,
                         const int32_t* run_chunks, const float* dht, void* dH, void* dR,
                         float* dh0, hipStream_t st, const int32_t* order) {
  const size_t sm1 = dh_smem<TI, D, CB>();
  GDN_BTRY(set_lds(k_bwd_dh<TI, D, CB>, sm1));
  k_bwd_dh<TI, D, CB><<<dim3(runs, p.H), dh_threads<D, CB>(), sm1, st>>>(
      b.st.table, run_chunks, static_cast<const TI*>(p.q), static_cast<const TI*>(p.k),
      static_cast<const TI*>(b.st.Tinv), p.beta, p.beta_f32 ? 1 : 0,
      static_cast<const TI*>(b.dO), b.st.g_t, dht, static_cast<TI*>(dH), static_cast<TI*>(dR),
      dh0, order, p.Ttot, p.H, p.Hg, p.scale);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t run_bwd_dh(const Problem& p, const BwdBuffers& b, int runs,
                      const int32_t* run_chunks, const float* dht, void* dH, void* dR,
                      float* dh0, hipStream_t st, const int32_t* order) {
  if (runs <= 0) return hipSuccess;
  if constexpr (sizeof(TI) == 2 && D == 128) {
    // two workgroups per CU pay off once the pairs outnumber the CUs several times over
    // (measured on 64 sequences x 64 heads: 7 % in index order, 1 % with the sequences
    // longest first; 512 or 256 pairs of equal length lose 4 and 13 %)
    int dev = 0, cus = 0;
    GDN_BTRY(hipGetDevice(&dev));
    GDN_BTRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    if ((long)runs * p.H >= 8L * (cus > 0 ? cus : 1))
      return run_bwd_dh_cb<TI, D, 2>(p, b, runs, run_chunks, dht, dH, dR, dh0, st, order);
  }
  return run_bwd_dh_cb<TI, D, 1>(p, b, runs, run_chunks, dht, dH, dR, dh0, st, order);
}

template <typename TI, int D>
hipError_t run_bwd_chunk(const Problem& p, const BwdBuffers& b, hipStream_t st) {
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const TI* dO = static_cast<const TI*>(b.dO);
  // grouped heads: one workgroup per (chunk, q/k head) runs the group's value heads
  const int gsz = p.H / p.Hg;
  const size_t sm2 = ChunkLds<TI, D>::bytes;
  const long items = (long)p.max_chunks * (gsz > 1 ? p.Hg : p.H);
  if (items == 0) return hipSuccess;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  auto launch = [&](auto kern) -> hipError_t {
    GDN_BTRY(set_lds(kern, sm2));
    // persistent: as many workgroups as stay resident at once, each walking items with the
    // grid as its stride
    int dev = 0, cus = 0, per_cu = 0;
    GDN_BTRY(hipGetDevice(&dev));
    GDN_BTRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    GDN_BTRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern,
                                                          chunk_threads<TI, D>(), sm2));
    const long slots = (long)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    const int grid = (int)(items < slots ? items : slots);
    kern<<<grid, chunk_threads<TI, D>(), sm2, st>>>(
        b.st.table, p.max_chunks, q, k, v, p.beta, p.beta_f32 ? 1 : 0, b.st.g_t,
        static_cast<const TI*>(b.st.h_c), static_cast<const TI*>(b.st.v_new),
        static_cast<const TI*>(b.dR), static_cast<const TI*>(b.dH), dO, b.dq, b.dk, b.dv,
        b.dg, b.dbeta, p.Hg, gsz, p.Ttot, p.H, p.Hg, p.scale, b.grad_bf16 ? 1 : 0);
    return hipGetLastError();
  };
  GDN_BTRY(gsz > 1 ? launch(k_bwd_chunk<TI, D, true>) : launch(k_bwd_chunk<TI, D, false>));
  return hipSuccess;
}

}  // namespace

bool bwd_supported(const Problem& p) {
  return p.f32 ? p.D == 64 : (p.D == 64 || p.D == 128);
}

hipError_t launch_bwd_dh(const Problem& p, const BwdBuffers& b, int runs,
                         const int32_t* run_chunks, const float* dht, void* dH, void* dR,
                         float* dh0, hipStream_t st, const int32_t* order) {
  if (p.f32) return run_bwd_dh<float, 64>(p, b, runs, run_chunks, dht, dH, dR, dh0, st, order);
  return p.D == 64
             ? run_bwd_dh<bf16, 64>(p, b, runs, run_chunks, dht, dH, dR, dh0, st, order)
             : run_bwd_dh<bf16, 128>(p, b, runs, run_chunks, dht, dH, dR, dh0, st, order);
}

hipError_t launch_bwd_chunk(const Problem& p, const BwdBuffers& b, hipStream_t st) {
  if (p.f32) return run_bwd_chunk<float, 64>(p, b, st);
  return p.D == 64 ? run_bwd_chunk<bf16, 64>(p, b, st) : run_bwd_chunk<bf16, 128>(p, b, st);
}

hipError_t launch_bwd(const Problem& p, const BwdBuffers& b, hipStream_t st) {
  GDN_BTRY(launch_bwd_dh(p, b, p.N, b.st.seq_chunks, b.dht, b.dH, b.dR, b.dh0, st, b.order));
  return launch_bwd_chunk(p, b, st);
}

}  // namespace gdn
