// Segmented variant: a long sequence split into S segments that run in parallel, for
// batches with too few (sequence, head) pairs to fill the GPU (the long-prompt case of the
// FlashQLA how-to, section 8.3).  The state recurrence is affine in the initial state:
//
//   h_end = M h_in + b,     M = the final state from h_in = I with v = 0,
//                           b = the final state from h_in = 0,
//
// (M is Dk x Dk and acts on the key index of h = S^T).  The fused kernel computes M and b
// for every segment in parallel; the kernels here build the segment table and compose the
// maps in order, h_in(s + 1) = M_s h_in(s) + b_s, after which a last fused pass over the
// segments, started from their true h_in, writes o.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "segment.h"

namespace gdn {

namespace {

__global__ void k_segment_table(int32_t* cu_seg, int N, int T, int S, int Ls) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i > N * S) return;
  if (i == N * S) {
    cu_seg[i] = N * T;
  } else {
    const int n = i / S, s = i - n * S;
    cu_seg[i] = n * T + min(s * Ls, T);
  }
}

// One workgroup per (sequence, head, 16-column slab of the state): the columns of
// h_out = M h_in + b are independent, so each slab is composed on its own.  h = h0 (zero
// when absent); for each segment s, h_in[n S + s] = h and h <- M[n S + s] h + b[n S + s];
// finally ht = h.  fp32 throughout.
//
// The product M h of a step is a D x D by D x 16 GEMM, done on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32): the slab is D / 16 output tiles of 16 x 16, spread over the four
// waves and kept in registers in the accumulator layout (lane l: rows 4 (l / 16) + i of
// column l % 16).  M is staged row-major in LDS and the slab column-major, both with a
// padded stride, so one float4 read per lane supplies four consecutive k of one row or
// column: matrix-core instruction j of a 16-wide k block takes k = k0 + 4 (l / 16) + j in
// lane l for both operands (any assignment of k to slots works as long as A and B agree).
// M is staged in row blocks of at most 128 rows (two for D = 256); the next row block, or
// the next step's first one and its b, is loaded into registers while a block is composed.
// One workgroup of 256 threads: thread i counts the segments of a contiguous run of
// sequences, a scan over the 256 partial sums gives every sequence's first segment, and
// each thread then writes its sequences' segment starts.
__global__ __launch_bounds__(256) void k_segment_table_packed(const int32_t* __restrict__ cu,
                                                              int32_t* __restrict__ cu_seg,
                                                              int32_t* __restrict__ seg_first,
                                                              int N, int Ttot, int Ls,
                                                              int nseg) {
  __shared__ int part[257];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256;
  const int n0 = min(tid * per, N), n1 = min(n0 + per, N);
  auto bound = [&](int i) { return min(max(cu[i], 0), Ttot); };
  int cnt = 0;
  for (int n = n0; n < n1; ++n) {
    const int bos = bound(n), eos = max(bound(n + 1), bos);
    cnt += (eos - bos + Ls - 1) / Ls;
  }
  part[tid + 1] = cnt;
  __syncthreads();
  if (tid == 0) {
    part[0] = 0;
    for (int i = 1; i <= 256; ++i) part[i] += part[i - 1];
  }
  __syncthreads();
  // every index is clamped to the planned nseg segments: a well-formed cu never reaches it,
  // a non-monotone one (unspecified results) must not write past the table either
  int first = min(part[tid], nseg);
  for (int n = n0; n < n1; ++n) {
    const int bos = bound(n), eos = max(bound(n + 1), bos);
    seg_first[n] = first;
    for (int t = bos; t < eos && first < nseg; t += Ls) cu_seg[first++] = t;
  }
  const int total = min(part[256], nseg);
  const int end = N > 0 ? max(bound(N), bound(0)) : 0;
  if (tid == 0) seg_first[N] = total;
  for (int i = total + tid; i <= nseg; i += 256) cu_seg[i] = end;
}

// REV: the backward's composition.  The gradient reaching a segment's start is affine in
// the gradient at its end, dh_in = M^T dh_end + e (M^T is the adjoint of the segment's state
// map; e the segment's own reverse pass from a zero end gradient).  The segments of each
// sequence are then taken last to first, M is read transposed, h0 is the sequence's dht and
// ht receives dh0; h_in[s] receives the gradient at segment s's end, and b holds e.
template <int D, bool REV = false>
__global__ __launch_bounds__(256) void k_segment_scan(const float* __restrict__ M,
                                                      const float* __restrict__ b,
                                                      const float* __restrict__ h0,
                                                      float* __restrict__ h_in,
                                                      float* __restrict__ ht,
                                                      const int32_t* __restrict__ seg_first,
                                                      int S, int H) {
  constexpr int RB = D > 128 ? 128 : D;  // rows of M staged in LDS at a time
  constexpr int NBLK = D / RB;           // row blocks per step (2 for D = 256)
  constexpr int NTB = RB / 16;           // output tiles per row block
  static_assert(NTB % 4 == 0, "the four waves take the same number of tiles");
  constexpr int TPB = NTB / 4;           // tiles per wave and row block
  constexpr int TPW = NBLK * TPB;        // tiles per wave
  constexpr int LD = D + 4;              // padded LDS stride (floats)
  constexpr int NV = RB * D / 4 / 256;   // float4 of a row block of M per thread
  static_assert(!REV || NBLK == 1, "the transposed composition stages M whole");
  __shared__ __align__(16) float ms[RB * LD];   // a row block of M: [row][k]
  __shared__ __align__(16) float hsT[16 * LD];  // h[k][col] stored as [col][k]
  const int nh = blockIdx.x, slab = blockIdx.y;
  const int n = nh / H, h = nh - n * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  const int col = 16 * slab + lc;
  const long DD = (long)D * D;
  const long hbase = ((long)n * H + h) * DD;
  const int s0 = seg_first ? seg_first[n] : n * S;
  const int ns = seg_first ? seg_first[n + 1] - s0 : S;  // this sequence's segments
  // step s takes segment s, or segment ns - 1 - s in reverse
  auto seg_off = [&](int s) { return (((long)s0 + (REV ? ns - 1 - s : s)) * H + h) * DD; };
  // accumulator u of a wave: row block u / TPB, tile wave + 4 (u % TPB) within it
  auto tile_of = [&](int u) { return (u / TPB) * NTB + wave + 4 * (u % TPB); };
  auto row_of = [&](int u, int i) { return 16 * tile_of(u) + 4 * lg + i; };

  f32x4 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[u][i] = h0 ? h0[hbase + (long)row_of(u, i) * D + col] : 0.f;

  // the next row block of M (of this step, or the first of the next step) and the next
  // step's b are loaded into registers while the current row block is composed
  f32x4 mreg[NV];  // native vectors: HIP's float4 struct is copied through memory
  f32x4 breg[TPW];
  if (ns > 0) {
    const long off = seg_off(0);
#pragma unroll
    for (int v = 0; v < NV; ++v)
      mreg[v] = *reinterpret_cast<const f32x4*>(&M[off + 4 * (tid + 256 * v)]);
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) breg[u][i] = b[off + (long)row_of(u, i) * D + col];
  }
  for (int s = 0; s < ns; ++s) {
    const long off = seg_off(s);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) h_in[off + (long)row_of(u, i) * D + col] = acc[u][i];
      *reinterpret_cast<f32x4*>(&hsT[lc * LD + 16 * tile_of(u) + 4 * lg]) = acc[u];
      acc[u] = breg[u];
    }
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int i = 4 * (tid + 256 * v);
        *reinterpret_cast<f32x4*>(&ms[(i / D) * LD + i % D]) = mreg[v];
      }
      __syncthreads();
      const bool next_step = bk + 1 == NBLK && s + 1 < ns;
      if (bk + 1 < NBLK || next_step) {
        const long moff = next_step ? seg_off(s + 1) : off + (long)(bk + 1) * RB * D;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          mreg[v] = *reinterpret_cast<const f32x4*>(&M[moff + 4 * (tid + 256 * v)]);
      }
      if (next_step) {
        const long boff = seg_off(s + 1);
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) breg[u][i] = b[boff + (long)row_of(u, i) * D + col];
      }
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 16) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&hsT[lc * LD + k0 + 4 * lg]);
#pragma unroll
        for (int j = 0; j < TPB; ++j) {
          const int u = bk * TPB + j;
          if constexpr (REV) {
            // M^T[row][k] = M[k][row]: four strided reads (rows 4 apart sit 16 banks apart)
            const float* pm = &ms[(k0 + 4 * lg) * LD + 16 * (wave + 4 * j) + lc];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(pm[q * LD], bv[q], acc[u], 0, 0, 0);
          } else {
            const f32x4 av = *reinterpret_cast<const f32x4*>(
                &ms[(16 * (wave + 4 * j) + lc) * LD + k0 + 4 * lg]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc[u], 0, 0, 0);
          }
        }
      }
      __syncthreads();  // ms (and, after the last block, hsT) is rewritten next
    }
  }
  if (ht) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) ht[hbase + (long)row_of(u, i) * D + col] = acc[u][i];
  }
}

// The first chunk (of the chunk table) of every segment, and the total at [nseg]: segment s
// of sequence n starts cps = Ls / C chunks after the previous one, clamped to the sequence's
// chunks; the planned segments past the last real one start (and end) at the total.
// Thread i takes sequence i (its segments) and table entry i past the real segments.
__global__ void k_segment_chunks(const int32_t* __restrict__ seq_chunks,
                                 const int32_t* __restrict__ seg_first,
                                 int32_t* __restrict__ seg_chunks, int N, int S, int cps,
                                 int nseg) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) {
    const int j0 = seg_first ? seg_first[i] : i * S, j1 = seg_first ? seg_first[i + 1] : j0 + S;
    const int c0 = seq_chunks[i], c1 = seq_chunks[i + 1];
    for (int j = j0; j < j1 && j < nseg; ++j)
      seg_chunks[j] = min(c0 + (j - j0) * cps, c1);
  }
  const int total = min(seg_first ? seg_first[N] : N * S, nseg);
  if (i >= total && i <= nseg) seg_chunks[i] = seq_chunks[N];
}

}  // namespace

hipError_t launch_segment_table(int32_t* cu_seg, int N, int T, int S, int Ls, hipStream_t st) {
  const int n = N * S + 1;
  k_segment_table<<<(n + 255) / 256, 256, 0, st>>>(cu_seg, N, T, S, Ls);
  return hipGetLastError();
}

hipError_t launch_segment_scan_ranges(const float* M, const float* b, const float* h0,
                                      float* h_in, float* ht, const int32_t* seg_first, int N,
                                      int S, int H, int D, hipStream_t st) {
  if (N * H == 0) return hipSuccess;
  const dim3 grid(N * H, D / 16);
  if (D == 64)
    k_segment_scan<64><<<grid, 256, 0, st>>>(M, b, h0, h_in, ht, seg_first, S, H);
  else if (D == 128)
    k_segment_scan<128><<<grid, 256, 0, st>>>(M, b, h0, h_in, ht, seg_first, S, H);
  else
    k_segment_scan<256><<<grid, 256, 0, st>>>(M, b, h0, h_in, ht, seg_first, S, H);
  return hipGetLastError();
}

hipError_t launch_segment_rscan(const float* M, const float* e, const float* dht,
                                float* dh_end, float* dh0, const int32_t* seg_first, int N,
                                int S, int H, int D, hipStream_t st) {
  if (N * H == 0) return hipSuccess;
  const dim3 grid(N * H, D / 16);
  if (D == 64)
    k_segment_scan<64, true><<<grid, 256, 0, st>>>(M, e, dht, dh_end, dh0, seg_first, S, H);
  else if (D == 128)
    k_segment_scan<128, true><<<grid, 256, 0, st>>>(M, e, dht, dh_end, dh0, seg_first, S, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_segment_chunks(const int32_t* seq_chunks, const int32_t* seg_first,
                                 int32_t* seg_chunks, int N, int S, int cps, int nseg,
                                 hipStream_t st) {
  const int n = (N > nseg + 1 ? N : nseg + 1);
  k_segment_chunks<<<(n + 255) / 256, 256, 0, st>>>(seq_chunks, seg_first, seg_chunks, N, S,
                                                     cps, nseg);
  return hipGetLastError();
}

hipError_t launch_segment_scan(const float* M, const float* b, const float* h0, float* h_in,
                               float* ht, int N, int S, int H, int D, hipStream_t st) {
  return launch_segment_scan_ranges(M, b, h0, h_in, ht, nullptr, N, S, H, D, st);
}

hipError_t launch_segment_table_packed(const int32_t* cu, int32_t* cu_seg, int32_t* seg_first,
                                       int N, int Ttot, int Ls, int nseg, hipStream_t st) {
  k_segment_table_packed<<<1, 256, 0, st>>>(cu, cu_seg, seg_first, N, Ttot, Ls, nseg);
  return hipGetLastError();
}

}  // namespace gdn
