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

// One workgroup per (sequence, head): h = h0 (zero when absent); for each segment s,
// h_in[n S + s] = h and h <- M[n S + s] h + b[n S + s]; finally ht = h.  fp32 throughout;
// thread (ty, tx) of a 16 x 16 grid owns rows ty R .. ty R + R - 1 and columns tx + 16 j
// (R = D / 16, j < R) of the D x D state, kept in LDS between steps.
template <int D>
__global__ __launch_bounds__(256) void k_segment_scan(const float* __restrict__ M,
                                                      const float* __restrict__ b,
                                                      const float* __restrict__ h0,
                                                      float* __restrict__ h_in,
                                                      float* __restrict__ ht, int S, int H) {
  constexpr int R = D / 16;
  __shared__ float hs[D * D];
  __shared__ float ms[D * D];
  const int n = blockIdx.x / H, h = blockIdx.x - n * H;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const long DD = (long)D * D;
  for (int i = tid; i < D * D; i += 256) hs[i] = h0 ? h0[((long)n * H + h) * DD + i] : 0.f;
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    const long off = (((long)n * S + s) * H + h) * DD;
    for (int i = tid; i < D * D; i += 256) {
      h_in[off + i] = hs[i];
      ms[i] = M[off + i];
    }
    __syncthreads();
    float acc[R][R];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < R; ++j) acc[r][j] = b[off + (long)(ty * R + r) * D + tx + 16 * j];
    for (int c = 0; c < D; ++c) {
      float x[R];
#pragma unroll
      for (int j = 0; j < R; ++j) x[j] = hs[c * D + tx + 16 * j];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float mv = ms[(ty * R + r) * D + c];
#pragma unroll
        for (int j = 0; j < R; ++j) acc[r][j] = fmaf(mv, x[j], acc[r][j]);
      }
    }
    __syncthreads();  // every read of hs and ms for this step is done
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < R; ++j) hs[(ty * R + r) * D + tx + 16 * j] = acc[r][j];
    __syncthreads();
  }
  if (ht)
    for (int i = tid; i < D * D; i += 256) ht[((long)n * H + h) * DD + i] = hs[i];
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
  if (D == 64)
    k_segment_scan<64><<<N * H, 256, 0, st>>>(M, b, h0, h_in, ht, S, H);
  else
    k_segment_scan<128><<<N * H, 256, 0, st>>>(M, b, h0, h_in, ht, S, H);
  return hipGetLastError();
}

}  // namespace gdn
