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
// finally ht = h.  fp32 throughout; thread (rg, c) owns column c of the slab and rows
// rg R .. rg R + R - 1 (R = D / 16), M is staged in LDS per step, the slab kept there.
template <int D>
__global__ __launch_bounds__(256) void k_segment_scan(const float* __restrict__ M,
                                                      const float* __restrict__ b,
                                                      const float* __restrict__ h0,
                                                      float* __restrict__ h_in,
                                                      float* __restrict__ ht, int S, int H) {
  constexpr int R = D / 16;
  __shared__ float hs[D * 16];
  constexpr int MS = D + 4;  // row stride of M in LDS (16-byte aligned rows, staggered banks)
  __shared__ __align__(16) float ms[D * MS];
  const int nh = blockIdx.x, slab = blockIdx.y;
  const int n = nh / H, h = nh - n * H;
  const int tid = threadIdx.x, c = tid % 16, rg = tid / 16;
  const int col = 16 * slab + c;
  const long DD = (long)D * D;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    acc[r] = h0 ? h0[((long)n * H + h) * DD + (long)(rg * R + r) * D + col] : 0.f;
  for (int s = 0; s < S; ++s) {
    const long off = (((long)n * S + s) * H + h) * DD;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = rg * R + r;
      h_in[off + (long)row * D + col] = acc[r];
      hs[row * 16 + c] = acc[r];
    }
    for (int i = 4 * tid; i < D * D; i += 4 * 256)
      *reinterpret_cast<float4*>(&ms[(i / D) * MS + i % D]) =
          *reinterpret_cast<const float4*>(&M[off + i]);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = b[off + (long)(rg * R + r) * D + col];
    for (int k = 0; k < D; k += 4) {
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = hs[(k + u) * 16 + c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4 mv = *reinterpret_cast<const float4*>(&ms[(rg * R + r) * MS + k]);
        acc[r] = fmaf(mv.x, x[0], acc[r]);
        acc[r] = fmaf(mv.y, x[1], acc[r]);
        acc[r] = fmaf(mv.z, x[2], acc[r]);
        acc[r] = fmaf(mv.w, x[3], acc[r]);
      }
    }
    __syncthreads();  // hs and ms are rewritten by the next step
  }
  if (ht)
#pragma unroll
    for (int r = 0; r < R; ++r) ht[((long)n * H + h) * DD + (long)(rg * R + r) * D + col] = acc[r];
}

}  // namespace

hipError_t launch_segment_table(int32_t* cu_seg, int N, int T, int S, int Ls, hipStream_t st) {
  const int n = N * S + 1;
  k_segment_table<<<(n + 255) / 256, 256, 0, st>>>(cu_seg, N, T, S, Ls);
  return hipGetLastError();
}

hipError_t launch_segment_scan(const float* M, const float* b, const float* h0, float* h_in,
                               float* ht, int N, int S, int H, int D, hipStream_t st) {
  if (N * H == 0) return hipSuccess;
  const dim3 grid(N * H, D / 16);
  if (D == 64)
    k_segment_scan<64><<<grid, 256, 0, st>>>(M, b, h0, h_in, ht, S, H);
  else
    k_segment_scan<128><<<grid, 256, 0, st>>>(M, b, h0, h_in, ht, S, H);
  return hipGetLastError();
}

}  // namespace gdn
