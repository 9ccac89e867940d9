// Host-side view of one call, shared by the C ABI (api.cpp) and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct Problem {
  int B, T, N, H, Hg, D, C;  // D = Dk = Dv
  int Ttot;                  // B * T tokens on the packed axis
  int max_chunks;            // ceil(Ttot / C) + N: bound on the number of chunks
  bool f32;                  // q, k, v, o are fp32 (else bf16)
  bool beta_f32;             // beta is fp32 (else bf16)
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;
  const int32_t* cu;
  void* o;
  float* ht;
  int fused_flags = 0;  // kFused* bits, for the passes of the segmented variant
  const int32_t* order = nullptr;  // packed batch: sequence of each workgroup rank, or NULL
  // Recurrent variant with the gates made in the kernel (the decode operator): raw per-token
  // inputs a (in place of g) and b (in beta, same dtype) and per-head A_log, dt_bias (fp32;
  // dt_bias may be NULL).  gate_a == NULL: g and beta are used as given.
  const void* gate_a = nullptr;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
  // Fused variant, D <= 128: also write each chunk's start state (bf16 [chunks][H][D][D],
  // chunk = seq_chunks[n] + m at 64-token chunks) and v_new (bf16 [Ttot][H][D]), for the
  // backward; hc_out == NULL: not written.
  const int32_t* seq_chunks = nullptr;
  void* hc_out = nullptr;
  void* vnew_out = nullptr;
};

// Fused-kernel modes used by the segmented variant's passes.
constexpr int kFusedZeroV = 1;       // v is read as zeros
constexpr int kFusedH0Identity = 2;  // h0 is the identity (Dk == Dv), not read from memory
constexpr int kFusedNoOutput = 4;    // o is not written

// Intermediates of the staged variant (device pointers inside the caller's workspace).
struct Stages {
  int32_t* table;       // [max_chunks][4]
  int32_t* seq_chunks;  // [N + 1]
  float* g_cum;         // [Ttot][H]
  float* g_t;           // [H][Ttot]
  void* beta_t;         // [H][Ttot]
  float* A;             // [Ttot][H][C]
  void* Tinv;           // [Ttot][H][C]
  void* W;              // [Ttot][H][D]
  void* U;              // [Ttot][H][D]
  void* h_c;            // [max_chunks][H][D][D]
  void* v_new;          // [Ttot][H][D]
};

// fuse_kkt_solve (C = 64, D <= 128): stages 3 and 4 as one launch that keeps A on chip (A is
// then not written); for callers that need only T, as the backward does.
hipError_t launch_staged(const Problem& p, const Stages& s, int stop_after, hipStream_t st,
                         bool fuse_kkt_solve = false);
// Stage 0 alone: the chunk table and each sequence's first chunk at p.C.
hipError_t launch_chunk_table(const Problem& p, const Stages& s, hipStream_t st);

// Backward pass: the forward's chunk quantities (chunk table, Gc, T at C = 64, each chunk's
// start state h_c and v_new; the staged layout) plus the gradient buffers.  dq, dk:
// [Ttot, Hg, D]; dv: [Ttot, H, D]; dg, dbeta: [Ttot, H]; dh0: [N, H, D, D] or NULL; all
// fp32.  dR [Ttot, H, D] and dH [max_chunks, H, D, D] (the gradient of each chunk's end
// state), in the q/k/v dtype, are workspace.
struct BwdBuffers {
  Stages st;
  const void* dO;
  const float* dht;
  void* dq;  // fp32, or bf16 when grad_bf16
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  void* dR;
  void* dH;
  const int32_t* order = nullptr;  // a packed batch's longest-first order, or null
  bool grad_bf16 = false;          // dq, dk, dv stored in bf16
};
bool bwd_supported(const Problem& p);
// Both backward kernels over the sequences (b.dht, b.dH, b.dR, b.dh0 as above).
hipError_t launch_bwd(const Problem& p, const BwdBuffers& b, hipStream_t st);
// The reverse pass alone over `runs` runs of consecutive chunks (sequences, or segments of
// them): run i covers chunks run_chunks[i] .. run_chunks[i + 1] - 1 of the chunk table and
// starts from dht[i] ([runs, H, D, D] fp32; zero when null); dh0[i] receives the gradient
// at its start (not written when null); dH and dR as above, not written when dH is null.
// With `order` (runs are a packed batch's sequences; order[rank] = sequence, longest first),
// the workgroups take the runs longest first, heads innermost.
hipError_t launch_bwd_dh(const Problem& p, const BwdBuffers& b, int runs,
                         const int32_t* run_chunks, const float* dht, void* dH, void* dR,
                         float* dh0, hipStream_t st, const int32_t* order = nullptr);
// The chunk-parallel kernel (with grouped heads, one workgroup runs a group's value heads).
hipError_t launch_bwd_chunk(const Problem& p, const BwdBuffers& b, hipStream_t st);
bool fused_supported(const Problem& p);
hipError_t launch_fused(const Problem& p, hipStream_t st);
// Longest-first order of a packed batch's sequences (order[rank] = sequence), for the fused
// kernel's workgroup ranks.
hipError_t launch_lpt_order(const int32_t* cu, int32_t* order, int N, int T, int Ttot,
                            hipStream_t st);
// Causal depthwise conv1d with a decode state (the step before the delta rule).
struct ConvProblem {
  int T, Ttot, N, C, W, lines;  // C channels (multiple of 8), W taps in {2, 3, 4}
  bool f32;                     // x, y, state are fp32 (else bf16)
  bool silu;
  const void* x;
  const float* weight;
  const float* bias;
  void* state;
  const int32_t* cache_indices;
  const int32_t* has_initial_state;
  const int32_t* cu;
  void* y;
};
hipError_t launch_conv1d(const ConvProblem& p, hipStream_t st);

// Recurrent variant: token by token, one wave per (sequence, head, 32 state columns).
hipError_t launch_recurrent(const Problem& p, hipStream_t st);
// Segmented variant: segment table (cu_seg[n S + s] = n T + min(s Ls, T), cu_seg[N S] =
// N T) and the sequential composition of the segments' affine state maps.
hipError_t launch_segment_table(int32_t* cu_seg, int N, int T, int S, int Ls, hipStream_t st);
hipError_t launch_segment_scan(const float* M, const float* b, const float* h0, float* h_in,
                               float* ht, int N, int S, int H, int D, hipStream_t st);

}  // namespace gdn
