// Causal depthwise 1-D convolution with a decode state, the step before the gated delta
// rule (the causal_conv1d operator of the TileLang × xLLM page: each output depends on the
// current and earlier tokens only, a per-sequence state line carries the last inputs from
// one call to the next, cache indices select the line, and a per-sequence flag says whether
// a sequence starts from its line or from zeros).
//
// For sequence n, channel c and position t of the sequence, with x~ = (the W - 1 inputs
// before the sequence: the state line, or zeros) followed by the sequence's inputs,
//
//   y[t, c] = act(bias[c] + sum_i weight[c, i] x~[t + i, c]),   i = 0 .. W - 1,
//
// and afterwards the line holds the last W - 1 entries of x~.  act is the identity or SiLU.
//
// Two launches.  k_conv1d: one thread per 8 consecutive channels (16 bytes of bf16) and a
// block of up to 64 consecutive tokens of the packed axis (fewer when that is needed to give
// the GPU enough workgroups), walked in order with the W - 1 previous inputs in registers;
// a wave reads 1 KiB of contiguous channels per token.  It only reads the state.
// k_conv_state then rewrites each sequence's line (one thread per 8 channels of a line), so
// a call may update the state in place even when several blocks of one sequence read it.
// When every sequence lies in one block (a dense batch of short sequences: decode), that
// block writes the line itself from its window and the second launch is skipped.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kVec = 8;         // channels per thread
constexpr int kThreads = 256;   // threads per workgroup: 2048 channels
constexpr int kMaxTokens = 64;  // tokens per thread, at most (fewer when that fills the GPU)
constexpr int kGroup = 8;       // tokens whose loads are issued together
constexpr int kFillGroups = 512;  // workgroups that keep 256 CUs busy (measured on decode)

template <typename E> struct Vec8;
template <> struct Vec8<bf16> {
  struct raw {
    bf16x8 a;
  };
  static __device__ __forceinline__ raw load_raw(const bf16* p) {
    return raw{*reinterpret_cast<const bf16x8*>(p)};
  }
  static __device__ __forceinline__ void wide(const raw& r, float* out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (float)r.a[i];
  }
  static __device__ __forceinline__ void load(const bf16* p, float* out) { wide(load_raw(p), out); }
  static __device__ __forceinline__ void store(bf16* p, const float* in) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (bf16)in[i];
    *reinterpret_cast<bf16x8*>(p) = x;
  }
};
template <> struct Vec8<float> {
  struct raw {
    float4 a, b;
  };
  static __device__ __forceinline__ raw load_raw(const float* p) {
    return raw{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  static __device__ __forceinline__ void wide(const raw& r, float* out) {
    out[0] = r.a.x; out[1] = r.a.y; out[2] = r.a.z; out[3] = r.a.w;
    out[4] = r.b.x; out[5] = r.b.y; out[6] = r.b.z; out[7] = r.b.w;
  }
  static __device__ __forceinline__ void load(const float* p, float* out) { wide(load_raw(p), out); }
  static __device__ __forceinline__ void store(float* p, const float* in) {
    reinterpret_cast<float4*>(p)[0] = make_float4(in[0], in[1], in[2], in[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(in[4], in[5], in[6], in[7]);
  }
};

struct ConvArgs {
  const void* x;
  const float* weight;  // [C, W]
  const float* bias;    // [C] or null
  void* state;          // [lines, W - 1, C] or null
  const int32_t* idx;   // [N] or null
  const int32_t* init;  // [N] or null
  const int32_t* cu;    // [N + 1] or null
  void* y;
  int T, Ttot, N, C, lines;
  int tokens;     // tokens per thread
  int own_state;  // every sequence lies in one token block: k_conv1d writes the lines
};

// Token range [bos, eos) of sequence n (cu values clamped to the token axis).
__device__ __forceinline__ void seq_bounds(const ConvArgs& a, int n, int& bos, int& eos) {
  if (a.cu) {
    bos = min(max(a.cu[n], 0), a.Ttot);
    eos = min(max(a.cu[n + 1], bos), a.Ttot);
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
}

// The state line sequence n starts from, or -1 (zeros: no state, the flag is 0, or the
// cache index lies outside [0, lines)).
__device__ __forceinline__ int start_line(const ConvArgs& a, int n) {
  if (!a.state || (a.init && a.init[n] == 0)) return -1;
  const int line = a.idx ? a.idx[n] : n;
  return (line >= 0 && line < a.lines) ? line : -1;
}

// The sequence that holds token t: the last n with start(n) <= t (dense: t / T).
__device__ __forceinline__ int find_seq(const ConvArgs& a, int t) {
  if (!a.cu) return t / a.T;
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(a.cu[mid], 0), a.Ttot) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int W, typename E, bool SILU>
__global__ __launch_bounds__(kThreads) void k_conv1d(ConvArgs a) {
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kVec;
  if (c0 >= a.C) return;
  const int t0 = blockIdx.x * a.tokens;
  const int tend = min(t0 + a.tokens, a.Ttot);
  const E* x = static_cast<const E*>(a.x);
  const E* st = static_cast<const E*>(a.state);
  E* y = static_cast<E*>(a.y);

  float w[W][kVec], b[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i][v] = a.weight[(long)(c0 + v) * W + i];
    b[v] = a.bias ? a.bias[c0 + v] : 0.f;
  }

  float win[W - 1][kVec];  // x~ at t - (W - 1) .. t - 1
  // After a sequence's last token the window is x~'s last W - 1 entries: its new line.
  // Only done when no other block reads the line (own_state).
  auto write_state = [&](int n) {
    const int line = a.idx ? a.idx[n] : n;
    if (line < 0 || line >= a.lines) return;
    E* sw = static_cast<E*>(a.state);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) Vec8<E>::store(sw + ((long)line * (W - 1) + j) * a.C + c0, win[j]);
  };
  // One output from the window and x[t]; then the window moves on by one token.
  auto emit = [&](int t, const float* xt) {
    float out[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      float z = fmaf(w[W - 1][v], xt[v], b[v]);
#pragma unroll
      for (int i = 0; i < W - 1; ++i) z = fmaf(w[i][v], win[i][v], z);
      if (SILU) z = z / (1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
      out[v] = z;
    }
    Vec8<E>::store(y + (long)t * a.C + c0, out);
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
#pragma unroll
      for (int i = 0; i + 1 < W - 1; ++i) win[i][v] = win[i + 1][v];
      win[W - 2][v] = xt[v];
    }
  };
  // The window for position t of sequence n (bounds bos, eos).
  auto fill = [&](int n, int t, int bos) {
    const int line = start_line(a, n);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int tau = t - (W - 1) + j;
      if (tau >= bos) {
        Vec8<E>::load(x + (long)tau * a.C + c0, win[j]);
      } else if (line >= 0) {
        Vec8<E>::load(st + ((long)line * (W - 1) + (W - 1) + (tau - bos)) * a.C + c0, win[j]);
      } else {
#pragma unroll
        for (int v = 0; v < kVec; ++v) win[j][v] = 0.f;
      }
    }
  };

  int n = find_seq(a, t0);
  int bos, eos;
  seq_bounds(a, n, bos, eos);
  if (t0 < eos && eos >= tend) {
    // the whole block lies in one sequence: loads issued kGroup tokens at a time
    fill(n, t0, bos);
    int t = t0;
    for (; t + kGroup <= tend; t += kGroup) {
      typename Vec8<E>::raw r[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) r[u] = Vec8<E>::load_raw(x + (long)(t + u) * a.C + c0);
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        float xt[kVec];
        Vec8<E>::wide(r[u], xt);
        emit(t + u, xt);
      }
    }
    for (; t < tend; ++t) {
      float xt[kVec];
      Vec8<E>::load(x + (long)t * a.C + c0, xt);
      emit(t, xt);
    }
    if (a.own_state && tend == eos) write_state(n);
    return;
  }
  bool fresh = true;
  for (int t = t0; t < tend; ++t) {
    while (t >= eos) {  // next non-empty sequence holding t
      if (++n >= a.N) return;  // tokens past the last sequence belong to none
      seq_bounds(a, n, bos, eos);
      fresh = true;
    }
    if (fresh) {
      fill(n, t, bos);
      fresh = false;
    }
    float xt[kVec];
    Vec8<E>::load(x + (long)t * a.C + c0, xt);
    emit(t, xt);
    if (a.own_state && t + 1 == eos) write_state(n);
  }
}

// New state lines: line(n)[j] = x~[len + j] for j < W - 1 (x~ = old line or zeros, then
// the sequence's inputs).  One thread per (sequence, 8 channels); it reads all W - 1 values
// before writing any, so the in-place shift of a short sequence is safe.
template <int W, typename E>
__global__ __launch_bounds__(kThreads) void k_conv_state(ConvArgs a) {
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  const int groups = a.C / kVec;
  if (gid >= (long)a.N * groups) return;
  const int n = (int)(gid / groups);
  const int c0 = (int)(gid - (long)n * groups) * kVec;
  const int line = a.idx ? a.idx[n] : n;
  if (line < 0 || line >= a.lines) return;
  const int from = start_line(a, n);  // == line, or -1 for a zero start
  int bos, eos;
  seq_bounds(a, n, bos, eos);
  const int len = eos - bos;
  const E* x = static_cast<const E*>(a.x);
  E* st = static_cast<E*>(a.state);
  float vals[W - 1][kVec];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int e = len + j;  // index into x~
    if (e >= W - 1) {
      Vec8<E>::load(x + (long)(bos + e - (W - 1)) * a.C + c0, vals[j]);
    } else if (from >= 0) {
      Vec8<E>::load(st + ((long)line * (W - 1) + e) * a.C + c0, vals[j]);
    } else {
#pragma unroll
      for (int v = 0; v < kVec; ++v) vals[j][v] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j) Vec8<E>::store(st + ((long)line * (W - 1) + j) * a.C + c0, vals[j]);
}

template <int W, typename E>
hipError_t launch_w(const ConvArgs& a, bool silu, hipStream_t s) {
  if (a.Ttot > 0) {
    const dim3 grid((a.Ttot + a.tokens - 1) / a.tokens, (a.C / kVec + kThreads - 1) / kThreads);
    if (silu)
      k_conv1d<W, E, true><<<grid, kThreads, 0, s>>>(a);
    else
      k_conv1d<W, E, false><<<grid, kThreads, 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state && a.N > 0 && !a.own_state) {
    const long threads = (long)a.N * (a.C / kVec);
    k_conv_state<W, E><<<(unsigned)((threads + kThreads - 1) / kThreads), kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const ConvArgs& a, int W, bool silu, hipStream_t s) {
  if (W == 2) return launch_w<2, E>(a, silu, s);
  if (W == 3) return launch_w<3, E>(a, silu, s);
  return launch_w<4, E>(a, silu, s);
}

}  // namespace

hipError_t launch_conv1d(const ConvProblem& p, hipStream_t s) {
  ConvArgs a;
  a.x = p.x;
  a.weight = p.weight;
  a.bias = p.bias;
  a.state = p.state;
  a.idx = p.cache_indices;
  a.init = p.has_initial_state;
  a.cu = p.cu;
  a.y = p.y;
  a.T = p.T;
  a.Ttot = p.Ttot;
  a.N = p.N;
  a.C = p.C;
  a.lines = p.lines;
  // the longest token block (a power of two up to kMaxTokens) that still gives kFillGroups
  // workgroups; decode batches get one token per thread
  const long slabs = (p.C / kVec + kThreads - 1) / kThreads;
  a.tokens = kMaxTokens;
  while (a.tokens > 1 && ((long)p.Ttot + a.tokens - 1) / a.tokens * slabs < kFillGroups)
    a.tokens >>= 1;
  // a dense batch whose sequence length divides the block: each sequence lies in one block,
  // which then also writes its line (one launch instead of two)
  a.own_state = p.state && !p.cu && p.T > 0 && a.tokens % p.T == 0;
  return p.f32 ? launch_e<float>(a, p.W, p.silu, s) : launch_e<bf16>(a, p.W, p.silu, s);
}

}  // namespace gdn
