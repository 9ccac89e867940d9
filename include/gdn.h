/*
 * libgdn — chunked Gated DeltaNet on AMD Instinct MI355X (gfx950): the forward pass, its
 * backward pass, the decode operator with in-kernel gates and the causal conv1d before it.
 *
 * The operation (one call): for every sequence n and value head h, with q/k head
 * hk = h / (H / Hg), starting from S = h0[n, h]^T (zero when h0 is NULL), for each token t
 *
 *     S   <- exp(g_t) S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t <- scale S q_t
 *
 * and finally ht[n, h] = S^T.  It is evaluated chunk by chunk (chunk length C) through
 * the seven stages of the MegaGDN-PTO page (section 1.1: cumsum, transpose,
 * scaled_dot_kkt, solve_tril, wy_fast, chunk_h, chunk_o), either as seven launches
 * (GDN_VARIANT_STAGED) or as one launch that keeps every intermediate on chip
 * (GDN_VARIANT_FUSED; the megakernel idea of the page's section 1.3).  GQA (Hg q/k heads
 * shared by H value heads in contiguous groups) follows the page's section 5.2, packed
 * variable-length batches via cu_seqlens its section 5.3, and the user-level call shape
 * (q, k, v, g, beta, scale, initial_state, output_final_state) the FlashQLA how-to, step 5.2.
 *
 * Layouts (all contiguous, row-major; the token axis of a packed batch is B = 1, T = total):
 *   q, k    [B, T, Hg, Dk]   qkv_dtype (bf16 or f32)
 *   v, o    [B, T, H,  Dv]   qkv_dtype
 *   g       [B, T, H]        f32, the log-decay (g <= 0 in the intended use)
 *   beta    [B, T, H]        beta_dtype (bf16 or f32)
 *   h0, ht  [N, H, Dk, Dv]   f32 (the [B, H, K, V] state layout of the FlashQLA how-to,
 *                            step 5.3): ht[n, h, a, b] = S[b, a]
 *   cu_seqlens [N + 1]       int32, device memory, cu[0] = 0, non-decreasing, cu[N] <= B*T
 *
 * Ownership: the caller allocates and frees every buffer (device memory) and the optional
 * workspace.  The library keeps no pointer after a call returns, allocates nothing, and
 * has no mutable global state; calls are reentrant.  All work is enqueued on `stream`
 * (NULL = the default stream) and nothing is synchronised: errors found on the host are
 * returned before any launch; a launch failure returns GDN_ERR_HIP.  cu_seqlens is read
 * only on the device: values outside [0, B*T] are clamped (a sequence never reads or
 * writes outside the token range), but non-monotone values give unspecified results.
 *
 * Input domain: any finite bf16 (or f32) q, k, v and h0 go through every variant without
 * overflow of an intermediate (the fused kernel's matrix-core operands are bf16, with
 * fp32's exponent range).  The accuracy stated for bf16 (relative L2 5e-3 on o, 1e-2 on ht)
 * assumes the workloads' keys, L2-normalised with beta in [0, 1] (beta |k|^2 <= 2: the
 * fused kernel forms the 16 x 16 diagonal inverses in fp16, whose factors are then
 * bounded), and g <= 0.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null required pointer, bad shape, misaligned pointer */
  GDN_ERR_UNSUPPORTED = 2, /* valid but not built: Dk != Dv, D not in {64,128,256}, ... */
  GDN_ERR_WORKSPACE = 3,   /* staged or segmented variant without the workspace it needs */
  GDN_ERR_HIP = 4          /* a HIP launch or attribute call failed */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_variant {
  GDN_VARIANT_AUTO = 0,      /* recurrent for a few tokens per sequence (dense: T <= 8;
                                packed: B*T <= 8 N); else fused when built for the shape,
                                otherwise staged; segmented for a batch of few long
                                sequences (dense or packed) when the workspace for it is
                                given (fused otherwise)                                    */
  GDN_VARIANT_STAGED = 1,    /* seven launches, intermediates in the workspace */
  GDN_VARIANT_FUSED = 2,     /* one launch, one workgroup per (sequence, head) */
  GDN_VARIANT_SEGMENTED = 3, /* every sequence split into segments that run in parallel
                                (dense: S per sequence; packed: ceil(len / Ls) per sequence,
                                the table built on the device).  The state recurrence is
                                affine in the initial state, h_end = M h_in + b; the fused
                                kernel finds M (from h_in = I, v = 0) and b (from h_in = 0)
                                of every segment, a scan composes h_in(s+1) = M_s h_in(s) +
                                b_s (fp32), and a last fused pass writes o.  Three passes over
                                the data, many-fold parallelism (the long-prompt case of the
                                FlashQLA how-to, section 8.3).  Needs the workspace reported
                                for it.                                                    */
  GDN_VARIANT_RECURRENT = 4  /* token by token, the state kept in registers: one read and one
                                write of each (sequence, head) state per call, whatever the
                                number of tokens, and one dependent step per token.  For
                                decode (one or a few tokens per sequence; the per-token
                                delta-rule kernel of the TileLang × xLLM page).  Any dtype
                                and D the header lists; no workspace; chunk is ignored.
                                ht may be the same buffer as h0 (state updated in place).
                                The gates arrive as g and beta, as in every variant.       */
} gdn_variant;

/* Intermediate buffers of the staged variant, readable through gdn_stage_buffer().  The
 * fused variant's stage stop (stop_after = 6 with GDN_VARIANT_FUSED) writes the chunk
 * table, the sequences' first chunks, h_c and v_new only, at its own 64-token chunk. */
typedef enum gdn_buffer {
  GDN_BUF_CHUNK_TABLE = 0, /* int32 [max_chunks, 4]: (sequence, first token, length, index
                              in sequence); unused rows have length 0                  */
  GDN_BUF_SEQ_CHUNKS = 1,  /* int32 [N + 1]: first chunk of each sequence; [N] = total    */
  GDN_BUF_G_CUM = 2,       /* f32 [B*T, H]: in-chunk inclusive prefix sum of g  (stage 1) */
  GDN_BUF_G_T = 3,         /* f32 [H, B*T]: g_cum transposed                    (stage 2) */
  GDN_BUF_BETA_T = 4,      /* beta_dtype [H, B*T]: beta transposed              (stage 2) */
  GDN_BUF_A = 5,           /* f32 [B*T, H, C]: gated strictly-lower K K^T       (stage 3) */
  GDN_BUF_TINV = 6,        /* qkv_dtype [B*T, H, C]: rows of (I + A)^-1         (stage 4) */
  GDN_BUF_W = 7,           /* qkv_dtype [B*T, H, Dk]                            (stage 5) */
  GDN_BUF_U = 8,           /* qkv_dtype [B*T, H, Dv]                            (stage 5) */
  GDN_BUF_H_C = 9,         /* qkv_dtype [max_chunks, H, Dk, Dv]: state at chunk start (6) */
  GDN_BUF_V_NEW = 10,      /* qkv_dtype [B*T, H, Dv]: U - W h_c                 (stage 6) */
  GDN_BUF_COUNT = 11
} gdn_buffer;

typedef struct gdn_desc {
  int32_t B, T;       /* dense batch [B, T, ...]; packed varlen: B = 1, T = total tokens */
  int32_t N;          /* sequences: B when cu_seqlens is NULL, else len(cu_seqlens) - 1 */
  int32_t H, Hg;      /* value heads, q/k heads; H % Hg == 0                              */
  int32_t Dk, Dv;     /* head dims; this build supports Dk == Dv in {64, 128, 256}        */
  int32_t chunk;      /* C in {64, 128} (0 selects 128): the chunk length of the staged
                         variant.  The fused and segmented variants run their own chunk
                         (64 tokens, 32 at D = 256: what three K/Q buffers allow in LDS) and
                         the recurrent one goes token by token, whatever C asks for; the
                         result is the same up to rounding (the chunked form is exact for
                         any chunk length).  gdn_resolved_chunk() reports the length run.  */
  int32_t qkv_dtype;  /* gdn_dtype of q, k, v, o                                          */
  int32_t beta_dtype; /* gdn_dtype of beta                                                */
  int32_t variant;    /* gdn_variant                                                      */
  int32_t stop_after; /* 0 = the whole pass.  Staged: k in 1..6 stops after stage k (the
                         page's section 7.4 debugging mode).  Fused: 6 only, and only for
                         bf16 with D in {64, 128}: the kernel keeps every stage on chip and
                         forms just the chunk-start states and v_new, which it then writes
                         to the workspace (GDN_BUF_H_C, GDN_BUF_V_NEW, at 64-token chunks)
                         instead of o; it never forms G, A, T, W or U, so 1..5 are refused
                         (GDN_ERR_UNSUPPORTED), as is any stop for the other variants.    */
  void* workspace;    /* device memory for the staged and segmented variants and the fused
                         variant's longest-first order (256-byte aligned; may be NULL for
                         fused, see gdn_chunk_fwd_workspace_size)                         */
  size_t workspace_bytes;
  int32_t grad_dtype; /* gdn_chunk_bwd only: gdn_dtype of dq, dk, dv.  GDN_F32 (0, the
                         default) or, with bf16 inputs, GDN_BF16 (the gradients rounded
                         once, at the store; half the bytes written).  Ignored by the
                         forward entry points.                                            */
} gdn_desc;

/* Causal depthwise 1-D convolution with a decode state: the step before the gated delta
 * rule (the causal_conv1d operator of the TileLang × xLLM page).  For sequence n, channel
 * c and position t of the sequence, with x~ = (the W - 1 inputs before the sequence, taken
 * from the sequence's state line, or zeros) followed by the sequence's inputs,
 *
 *     y[t, c] = act(bias[c] + sum_{i < W} weight[c, i] x~[t + i, c])
 *
 * (weight[c, W - 1] multiplies the current token) and, when conv_state is given, the line
 * afterwards holds the last W - 1 entries of x~ (part of the old line when the sequence is
 * shorter than W - 1).  act is the identity or SiLU (z sigmoid(z)), in fp32.
 *
 * Layouts (contiguous, row-major; channels contiguous so that a token's row is one read):
 *   x, y        [B, T, C]            dtype (bf16 or f32); packed: B = 1, T = total tokens
 *   weight      [C, W]               f32
 *   bias        [C]                  f32, or NULL (zero)
 *   conv_state  [state_lines, W - 1, C]  dtype, or NULL (zeros in, nothing written); read
 *                                    and written in place
 *   cache_indices      [N] int32 or NULL (sequence n uses line n): an index outside
 *                      [0, state_lines) gives a zero start and leaves every line untouched
 *   has_initial_state  [N] int32 or NULL (all start from their line): 0 = start from zeros
 *   cu_seqlens         [N + 1] int32 or NULL (dense batch), as for gdn_chunk_fwd
 * C is a multiple of 8 and W is 2, 3 or 4; pointers are device pointers, x, y and conv_state
 * 16-byte aligned; weight is required, x and y too unless B*T = 0.  Two sequences naming the same line give unspecified lines.  Errors are
 * returned before any launch; the work is enqueued on `stream` (two launches: outputs, then
 * the state lines). */
typedef enum gdn_activation { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_activation;

typedef struct gdn_conv_desc {
  int32_t B, T;        /* dense [B, T, C]; packed: B = 1, T = total tokens              */
  int32_t N;           /* sequences: B (or 0) for a dense batch, len(cu_seqlens) - 1     */
  int32_t channels;    /* C                                                             */
  int32_t width;       /* W                                                             */
  int32_t dtype;       /* gdn_dtype of x, y and conv_state                              */
  int32_t activation;  /* gdn_activation                                                */
  int32_t state_lines; /* lines in conv_state                                           */
} gdn_conv_desc;

gdn_status gdn_causal_conv1d_fwd(const gdn_conv_desc* d, const void* x, const float* weight,
                                 const float* bias, void* conv_state,
                                 const int32_t* cache_indices,
                                 const int32_t* has_initial_state, const int32_t* cu_seqlens,
                                 void* y, hipStream_t stream);

/* Bytes of workspace the variant chosen by d->variant needs (for AUTO, what AUTO picks when
 * given that much).  The fused variant needs none on a dense batch; on a packed batch of
 * 2 .. 65536 sequences it asks for 4 bytes per sequence (256-byte aligned) to run them
 * longest first (an order kernel ranks them by length; the last workgroups to start are then
 * the shortest).  Given less, it runs them in index order: the same results, bit for bit.  The query cannot see cu_seqlens: a
 * descriptor with N other than 0 or B is a packed batch, one with B == 1 may be either and
 * gets the larger of the two needs, any other is a dense batch.  Host-only, no device work.
 * Returns 0 and sets *status on an invalid descriptor. */
size_t gdn_chunk_fwd_workspace_size(const gdn_desc* d, gdn_status* status);

/* The gdn_variant that gdn_chunk_fwd(d, ..., cu_seqlens, ...) runs with this descriptor and
 * workspace (AUTO resolved), or -1 if the call would be refused.  Only the nullness of
 * cu_seqlens is used; host-only, no device work. */
int32_t gdn_resolved_variant(const gdn_desc* d, const int32_t* cu_seqlens);

/* The chunk length gdn_chunk_fwd(d, ..., cu_seqlens, ...) runs with this descriptor: C for
 * the staged variant, the fused kernel's own chunk for the fused and segmented ones, 1 for
 * the recurrent one; -1 if the call would be refused.  Host-only, no device work. */
int32_t gdn_resolved_chunk(const gdn_desc* d, const int32_t* cu_seqlens);

/* The forward pass.  q, k, v, g, beta, o are required unless B*T = 0 (then every sequence
 * is empty: ht = h0, or zeros, and nothing else is touched, whatever the variant); h0 (zero
 * state), cu_seqlens (dense batch) and ht (final state not written) may be NULL.  scale multiplies o (Dk^-0.5 is the
 * usual choice).  Pointers must be device pointers aligned to 16 bytes (g, beta, cu_seqlens:
 * 4 / 2 / 4 bytes).  With stop_after = k > 0 (staged, or fused with k = 6) o and ht are
 * not written. */
gdn_status gdn_chunk_fwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* h0,
                         const int32_t* cu_seqlens, float scale, void* o, float* ht,
                         hipStream_t stream);

/* The decode operator with its gates made in the kernel (fused_sigmoid_gating_delta_rule,
 * the TileLang × xLLM page's section on the three core operators: the sigmoid activation,
 * the gate computation from A_log, the decay rate, and the delta-rule state update in one
 * kernel).  The page prints no formula; the reading is, per token t and value head h,
 *
 *     g_t    = -exp(A_log[h]) * softplus(a_t + dt_bias[h]),   softplus(x) = log(1 + e^x)
 *     beta_t = sigmoid(b_t) = 1 / (1 + e^-b_t)
 *
 * followed by exactly the recurrence of gdn_chunk_fwd with these g and beta, token by token
 * (the recurrent variant's kernel, the gates made in fp32 in the same kernel).
 *   a, b        [B, T, H]   d->beta_dtype (bf16 or f32): raw gate and beta inputs
 *   A_log       [H] f32     log of each head's decay rate (required)
 *   dt_bias     [H] f32     added to a before softplus, or NULL (zero)
 * Every other argument, layout and rule as for gdn_chunk_fwd (h0 and ht may be the same
 * buffer: the state is then updated in place, as a decode loop wants).  d->variant must be
 * GDN_VARIANT_AUTO or GDN_VARIANT_RECURRENT (else GDN_ERR_UNSUPPORTED); d->chunk is
 * ignored; no workspace. */
gdn_status gdn_fused_sigmoid_gating_delta_rule(const gdn_desc* d, const void* q, const void* k,
                                               const void* v, const void* a, const void* b,
                                               const float* A_log, const float* dt_bias,
                                               const float* h0, const int32_t* cu_seqlens,
                                               float scale, void* o, float* ht,
                                               hipStream_t stream);

/* How gdn_chunk_bwd(d, ..., cu_seqlens, ...) runs with this descriptor:
 * GDN_VARIANT_SEGMENTED (both sequential passes per segment), GDN_VARIANT_FUSED (the fused
 * kernel's recompute, one reverse pass per sequence), GDN_VARIANT_STAGED (the staged
 * recompute: f32), or -1 if the call would be refused.  Only the nullness of cu_seqlens is
 * used; host-only, no device work. */
int32_t gdn_chunk_bwd_resolved_variant(const gdn_desc* d, const int32_t* cu_seqlens);

/* Bytes of workspace gdn_chunk_bwd needs for this descriptor (N other than 0 or B reads as a
 * packed batch of N sequences, anything else as B dense sequences).  Host-only, no device
 * work.  Returns 0 and sets *status on an invalid or unsupported descriptor. */
size_t gdn_chunk_bwd_workspace_size(const gdn_desc* d, gdn_status* status);

/* The backward pass of gdn_chunk_fwd (the FlashQLA how-to reports forward and backward
 * speed-ups of the chunked operator, section 4.3; none of the pages prints the backward's
 * formulas).  Given the forward's inputs and the gradients of its outputs, it writes the
 * gradients of its inputs: the exact derivative of the recurrence, computed chunk by chunk
 * (C = 64) from the forward's chunk quantities, which it recomputes into the workspace
 * (nothing of a forward call is kept): T = (I + A)^-1 by the staged stages 0-4, then the
 * chunk-start states and v_new by the fused kernel (bf16), or stages 5-6 (f32).  The
 * gradients of the chunk-end states then run back through each sequence's chunks in order.
 * Few long sequences (AUTO: when segmenting pays, as for gdn_chunk_fwd's segmented variant;
 * GDN_VARIANT_SEGMENTED: always, bf16 only) run both sequential passes per segment: the
 * states from the segmented forward's maps, and the gradients by the adjoint map (a
 * segment's start gradient is M^T times its end gradient plus its own share), composed last
 * to first.  Any other variant keeps one pass per sequence.
 *   dout  [B, T, H, Dv]   qkv_dtype   gradient of o (required)
 *   dht   [N, H, Dk, Dv]  f32         gradient of ht, or NULL (zero)
 *   dq, dk [B, T, Hg, Dk] grad_dtype  the q/k heads' gradients (summed over the value heads
 *                                     that share them; fp32 sums, rounded once at the store)
 *   dv    [B, T, H, Dv]   grad_dtype
 *   dg, dbeta [B, T, H]   f32
 *   dh0   [N, H, Dk, Dv]  f32         gradient of h0, or NULL (not written)
 * Inputs, scale, cu_seqlens and their layouts as for gdn_chunk_fwd (h0 NULL = zero state).
 * Supported: bf16 with Dk = Dv in {64, 128}; f32 with Dk = Dv = 64; d->grad_dtype GDN_F32, or
 * GDN_BF16 with bf16 inputs (else GDN_ERR_UNSUPPORTED; another value: GDN_ERR_INVALID_ARG).  d->chunk and d->stop_after are ignored.  The workspace
 * (d->workspace, 256-byte aligned, gdn_chunk_bwd_workspace_size bytes) is required when
 * B*T > 0, else GDN_ERR_WORKSPACE.  Results do not depend on scheduling (no atomics).
 * Pointers are device pointers aligned to 16 bytes (g, beta, dg, dbeta, cu_seqlens: 4 / 2 /
 * 4 / 4 / 4).  With B*T = 0 only dh0 is written (= dht, or zeros). */
gdn_status gdn_chunk_bwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* h0,
                         const int32_t* cu_seqlens, float scale, const void* dout,
                         const float* dht, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* dh0, hipStream_t stream);

/* Bytes of device scratch the library holds on each GPU for gdn_chunk_fwd_noalloc. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid it.  Same
 * arguments, checks and results as gdn_chunk_fwd, except that d->workspace and
 * d->workspace_bytes are ignored: the workspace is the library's own scratch, a static
 * device array of GDN_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends (its address is looked up on the first call on a device).  A variant
 * that needs more returns GDN_ERR_WORKSPACE; AUTO picks among what fits, as it does for
 * any workspace.  Nothing is allocated and nothing needs clearing between calls.  Every
 * call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * other host threads) race and give unspecified results.  stop_after must be 0
 * (GDN_ERR_INVALID_ARG otherwise): stage buffers in the scratch are out of the caller's
 * reach. */
gdn_status gdn_chunk_fwd_noalloc(const gdn_desc* d, const void* q, const void* k,
                                 const void* v, const float* g, const void* beta,
                                 const float* h0, const int32_t* cu_seqlens, float scale,
                                 void* o, float* ht, hipStream_t stream);

/* Where intermediate `buf` lives inside the workspace of a stage-stop call (offset and size
 * in bytes), for stage-by-stage inspection (the page's section 7.4 debugging mode): the
 * staged layout at C, or, for GDN_VARIANT_FUSED with stop_after = 6, the fused stop's
 * layout at 64-token chunks, where the buffers it does not write have size 0. */
gdn_status gdn_stage_buffer(const gdn_desc* d, int32_t buf, size_t* offset, size_t* bytes);

/* Static, human-readable text for a status code. */
const char* gdn_status_string(gdn_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
