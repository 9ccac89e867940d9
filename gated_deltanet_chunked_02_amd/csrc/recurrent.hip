// Recurrent variant: the gated delta rule evaluated token by token, for batches with few
// tokens per sequence (decode, where the TileLang × xLLM page runs its fused sigmoid-gating
// delta-rule kernel once per token).  The chunked form's block work buys nothing there: each
// (sequence, head) costs one read and one write of its Dk x Dv fp32 state whatever the
// number of tokens, so the kernel is bound by HBM on the state and keeps it in registers
// between tokens.
//
// With the state held as H = S^T (Dk x Dv, row a = key index, column j = value index), one
// token is, for every column j,
//
//   s_j = k . H[:, j],   r_j = q . H[:, j]                     (before the update)
//   u_j = beta (v_j - e s_j),   e = exp(g)
//   H[:, j] <- e H[:, j] + u_j k
//   o_j = scale q . H[:, j] = scale (e r_j + (q . k) u_j)
//
// which is S <- e S (I - beta k k^T) + beta v k^T followed by o = scale S q, the gated
// delta rule of the MegaGDN-PTO page's section 1.1, written per column of H.
//
// GATED: the decode operator of the TileLang × xLLM page (fused_sigmoid_gating_delta_rule)
// also makes the gates in the kernel, from the raw per-token inputs a and b and the per-head
// A_log and dt_bias: g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b), in fp32,
// with softplus(x) = max(x, 0) + log1p(e^-|x|) (no overflow).
//
// Mapping: one wave per (sequence, head, 32-column slab of H).  Lane l = 8 rg + cg holds the
// four columns 4 cg .. 4 cg + 3 of the slab for the R = D / 8 rows rg R .. rg R + R - 1, so a
// row's 32 columns are 128 contiguous bytes read by 8 lanes.  The sums over the key index
// are reduced across the 8 row groups with three butterfly exchanges; no LDS, no barrier.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kSlab = 32;  // columns of H per wave

// Four consecutive elements: loaded raw (so a load for the next token can stay in flight
// while the current one is computed), widened to fp32 when used.
template <typename E> struct Vec4;
template <> struct Vec4<float> {
  typedef float4 raw;
  static __device__ __forceinline__ raw load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ float4 wide(raw x) { return x; }
  static __device__ __forceinline__ void store(float* p, float4 x) {
    *reinterpret_cast<float4*>(p) = x;
  }
};
template <> struct Vec4<bf16> {
  typedef bf16x4 raw;
  static __device__ __forceinline__ raw load(const bf16* p) {
    return *reinterpret_cast<const bf16x4*>(p);
  }
  static __device__ __forceinline__ float4 wide(raw x) {
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  }
  static __device__ __forceinline__ void store(bf16* p, float4 x) {
    const bf16x4 y = {(bf16)x.x, (bf16)x.y, (bf16)x.z, (bf16)x.w};
    *reinterpret_cast<bf16x4*>(p) = y;
  }
};

// The inputs of one token as one lane needs them: its R rows of k and q, its four columns
// of v, and the token's gate and beta (GATED: the raw inputs a and b, in beta's dtype).
template <int R, typename E, bool GATED> struct TokenIn {
  typename Vec4<E>::raw k[R / 4], q[R / 4], v;
  float g, b;

  __device__ __forceinline__ void load(const E* __restrict__ qp, const E* __restrict__ kp,
                                       const E* __restrict__ vp, const void* __restrict__ gp,
                                       const void* __restrict__ bp, int beta_f32, long qk_off,
                                       long v_off, long gi) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      k[i] = Vec4<E>::load(kp + qk_off + 4 * i);
      q[i] = Vec4<E>::load(qp + qk_off + 4 * i);
    }
    v = Vec4<E>::load(vp + v_off);
    g = GATED ? load_beta(gp, beta_f32, gi) : static_cast<const float*>(gp)[gi];
    b = load_beta(bp, beta_f32, gi);
  }
};

// Sum over the 8 lanes that share cg (lane bits 3..5).
__device__ __forceinline__ float row_group_sum(float x) {
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int D, typename E, bool GATED>
__global__ __launch_bounds__(64) void k_recurrent(const E* __restrict__ q,
                                                  const E* __restrict__ k,
                                                  const E* __restrict__ v,
                                                  const void* __restrict__ g,
                                                  const void* __restrict__ beta, int beta_f32,
                                                  const float* __restrict__ A_log,
                                                  const float* __restrict__ dt_bias,
                                                  const float* __restrict__ h0,
                                                  const int32_t* __restrict__ cu,
                                                  E* __restrict__ o, float* __restrict__ ht,
                                                  int T, int Ttot, int H, int Hg, float scale) {
  constexpr int R = D / 8;
  constexpr int NS = D / kSlab;
  const int wid = blockIdx.x;
  const int slab = wid % NS;
  const int nh = wid / NS;
  const int n = nh / H, h = nh - n * H;
  const int hk = h / (H / Hg);
  const int lane = threadIdx.x;
  const int rg = lane >> 3, cg = lane & 7;
  const int row0 = rg * R;
  const int col = slab * kSlab + 4 * cg;

  // GATED: the head's decay rate exp(A_log) and step-size bias
  float rate = 0.f, dtb = 0.f;
  if constexpr (GATED) {
    rate = __expf(A_log[h]);
    if (dt_bias) dtb = dt_bias[h];
  }

  int bos, eos;
  if (cu) {
    bos = min(max(cu[n], 0), Ttot);
    eos = min(max(cu[n + 1], bos), Ttot);
  } else {
    bos = n * T;
    eos = bos + T;
  }

  const long sbase = (long)nh * D * D;
  float4 st[R];
  if (h0) {
#pragma unroll
    for (int r = 0; r < R; ++r) st[r] = *reinterpret_cast<const float4*>(h0 + sbase + (long)(row0 + r) * D + col);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) st[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // token t's inputs are in `cur`; token t + 1's are loaded while t is computed
  auto qk_off = [&](int t) { return ((long)t * Hg + hk) * D + row0; };
  auto v_off = [&](int t) { return ((long)t * H + h) * D + col; };
  TokenIn<R, E, GATED> cur;
  if (bos < eos) cur.load(q, k, v, g, beta, beta_f32, qk_off(bos), v_off(bos), (long)bos * H + h);
  for (int t = bos; t < eos; ++t) {
    TokenIn<R, E, GATED> nxt;
    if (t + 1 < eos)
      nxt.load(q, k, v, g, beta, beta_f32, qk_off(t + 1), v_off(t + 1), (long)(t + 1) * H + h);
    float kr[R], qr[R];
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      const float4 a = Vec4<E>::wide(cur.k[i]);
      const float4 b = Vec4<E>::wide(cur.q[i]);
      kr[4 * i] = a.x; kr[4 * i + 1] = a.y; kr[4 * i + 2] = a.z; kr[4 * i + 3] = a.w;
      qr[4 * i] = b.x; qr[4 * i + 1] = b.y; qr[4 * i + 2] = b.z; qr[4 * i + 3] = b.w;
    }
    const float4 vt = Vec4<E>::wide(cur.v);
    float gl = cur.g, bt = cur.b;
    if constexpr (GATED) {
      const float x = cur.g + dtb;
      gl = -rate * (fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));  // -exp(A_log) softplus(x)
      bt = 1.f / (1.f + __expf(-cur.b));                         // sigmoid(b)
    }
    const float e = __builtin_amdgcn_exp2f(gl * 1.4426950408889634f);  // exp(g)

    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f, qk = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s0 = fmaf(kr[r], st[r].x, s0);
      s1 = fmaf(kr[r], st[r].y, s1);
      s2 = fmaf(kr[r], st[r].z, s2);
      s3 = fmaf(kr[r], st[r].w, s3);
      r0 = fmaf(qr[r], st[r].x, r0);
      r1 = fmaf(qr[r], st[r].y, r1);
      r2 = fmaf(qr[r], st[r].z, r2);
      r3 = fmaf(qr[r], st[r].w, r3);
      qk = fmaf(qr[r], kr[r], qk);
    }
    s0 = row_group_sum(s0);
    s1 = row_group_sum(s1);
    s2 = row_group_sum(s2);
    s3 = row_group_sum(s3);
    r0 = row_group_sum(r0);
    r1 = row_group_sum(r1);
    r2 = row_group_sum(r2);
    r3 = row_group_sum(r3);
    qk = row_group_sum(qk);

    const float u0 = bt * (vt.x - e * s0);
    const float u1 = bt * (vt.y - e * s1);
    const float u2 = bt * (vt.z - e * s2);
    const float u3 = bt * (vt.w - e * s3);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      st[r].x = fmaf(e, st[r].x, u0 * kr[r]);
      st[r].y = fmaf(e, st[r].y, u1 * kr[r]);
      st[r].z = fmaf(e, st[r].z, u2 * kr[r]);
      st[r].w = fmaf(e, st[r].w, u3 * kr[r]);
    }
    if (rg == 0) {
      const float4 ot = make_float4(scale * fmaf(e, r0, qk * u0), scale * fmaf(e, r1, qk * u1),
                                    scale * fmaf(e, r2, qk * u2), scale * fmaf(e, r3, qk * u3));
      Vec4<E>::store(o + v_off(t), ot);
    }
    if (t + 1 < eos) cur = nxt;  // nxt was loaded only when a next token exists
  }

  if (ht) {
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<float4*>(ht + sbase + (long)(row0 + r) * D + col) = st[r];
  }
}

template <int D, typename E, bool GATED>
hipError_t launch_g(const Problem& p, hipStream_t st) {
  const long waves = (long)p.N * p.H * (D / kSlab);
  k_recurrent<D, E, GATED><<<dim3((unsigned)waves), dim3(64), 0, st>>>(
      static_cast<const E*>(p.q), static_cast<const E*>(p.k), static_cast<const E*>(p.v),
      GATED ? p.gate_a : static_cast<const void*>(p.g), p.beta, p.beta_f32 ? 1 : 0, p.A_log,
      p.dt_bias, p.h0, p.cu, static_cast<E*>(p.o), p.ht, p.T, p.Ttot, p.H, p.Hg, p.scale);
  return hipGetLastError();
}

template <int D, typename E>
hipError_t launch_d(const Problem& p, hipStream_t st) {
  return p.gate_a ? launch_g<D, E, true>(p, st) : launch_g<D, E, false>(p, st);
}

template <typename E>
hipError_t launch_e(const Problem& p, hipStream_t st) {
  if (p.D == 64) return launch_d<64, E>(p, st);
  if (p.D == 128) return launch_d<128, E>(p, st);
  return launch_d<256, E>(p, st);
}

}  // namespace

hipError_t launch_recurrent(const Problem& p, hipStream_t st) {
  if ((long)p.N * p.H == 0) return hipSuccess;
  return p.f32 ? launch_e<float>(p, st) : launch_e<bf16>(p, st);
}

}  // namespace gdn
