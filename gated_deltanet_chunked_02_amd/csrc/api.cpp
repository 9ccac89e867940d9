// C ABI of libgdn (declared in include/gdn.h): host-side validation, the staged
// workspace layout and dispatch to the launchers.  No allocation, no synchronisation.
#include <stdint.h>
#include <string.h>

#include "gdn.h"
#include "gdn_internal.h"
#include "segment.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Layout {
  size_t off[GDN_BUF_COUNT];
  size_t bytes[GDN_BUF_COUNT];
  size_t total;
};

// Shape checks shared by every entry point; fills the shape part of the problem.
gdn_status check_desc(const gdn_desc* d, gdn::Problem* p) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->B < 1 || d->T < 0 || d->N < 0 || d->H < 1 || d->Hg < 1 || d->Dk < 1 || d->Dv < 1)
    return GDN_ERR_INVALID_ARG;
  if (d->H % d->Hg != 0) return GDN_ERR_INVALID_ARG;
  if (d->qkv_dtype != GDN_F32 && d->qkv_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->beta_dtype != GDN_F32 && d->beta_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->variant < GDN_VARIANT_AUTO || d->variant > GDN_VARIANT_RECURRENT)
    return GDN_ERR_INVALID_ARG;
  if (d->stop_after < 0 || d->stop_after > 6) return GDN_ERR_INVALID_ARG;
  const int C = d->chunk == 0 ? 128 : d->chunk;
  if (C != 64 && C != 128) return GDN_ERR_UNSUPPORTED;
  if (d->Dk != d->Dv) return GDN_ERR_UNSUPPORTED;
  const int D = d->Dk;
  if (D != 64 && D != 128 && D != 256) return GDN_ERR_UNSUPPORTED;
  const bool f32 = d->qkv_dtype == GDN_F32;
  const long long Ttot = (long long)d->B * d->T;
  if (Ttot > (1LL << 30)) return GDN_ERR_UNSUPPORTED;
  const int N = d->N == 0 ? d->B : d->N;
  if (N > (1 << 24)) return GDN_ERR_UNSUPPORTED;
  p->B = d->B;
  p->T = d->T;
  p->N = N;
  p->H = d->H;
  p->Hg = d->Hg;
  p->D = D;
  p->C = C;
  p->Ttot = (int)Ttot;
  p->max_chunks = (int)((Ttot + C - 1) / C) + N;
  p->f32 = f32;
  p->beta_f32 = d->beta_dtype == GDN_F32;
  return GDN_OK;
}

// Segments of the segmented variant: segments of Ls tokens (a multiple of the fused kernel's
// 64-token chunk; the last of a sequence may be shorter).  A dense batch has S per sequence
// (nseg = N S); a packed batch has ceil(len / Ls) per sequence, at most nseg in total.
struct SegPlan {
  bool use = false;  // AUTO: segmenting pays off (a forced request always segments)
  bool packed = false;
  int S = 1, Ls = 0;
  long nseg = 0;
};

constexpr int kFusedChunk = 64;
constexpr int kTargetPairs = 256;    // (segment, head) pairs that fill the GPU: one per CU
constexpr int kAutoMinSegments = 4;  // AUTO segments only when it gives at least 4 segments
constexpr int kAutoMinSegLen = 512;  // of at least 512 tokens (three passes over the data)

SegPlan seg_plan_packed(const gdn::Problem& p, bool forced) {
  // about kTargetPairs (segment, head) pairs over the whole token axis
  SegPlan sp;
  sp.packed = true;
  const long pairs = (long)p.N * p.H;
  long Ls = ((long)p.Ttot * p.H + kTargetPairs - 1) / kTargetPairs;
  Ls = (Ls + kFusedChunk - 1) / kFusedChunk * kFusedChunk;
  if (Ls < kFusedChunk) Ls = kFusedChunk;
  sp.Ls = (int)Ls;
  sp.nseg = ((long)p.Ttot + Ls - 1) / Ls + p.N;
  // AUTO: the sequences do not fill the GPU, and they average at least kAutoMinSegments
  // segments of at least kAutoMinSegLen tokens
  sp.use = forced || (pairs < kTargetPairs && Ls >= kAutoMinSegLen &&
                      (long)p.Ttot >= (long)kAutoMinSegments * p.N * Ls);
  return sp;
}

SegPlan seg_plan(const gdn::Problem& p, bool forced, bool dense) {
  if (!dense) return seg_plan_packed(p, forced);
  SegPlan sp;
  sp.use = forced;
  sp.nseg = p.N;
  const long pairs = (long)p.N * p.H;
  if (pairs <= 0 || p.T <= 0) return sp;
  const long want = (kTargetPairs + pairs - 1) / pairs;
  const long maxs = (p.T + kFusedChunk - 1) / kFusedChunk;
  long S = want < maxs ? want : maxs;
  if (S < 1) S = 1;
  long Ls = (p.T + S - 1) / S;
  Ls = (Ls + kFusedChunk - 1) / kFusedChunk * kFusedChunk;
  S = (p.T + Ls - 1) / Ls;
  if (!forced && (S < kAutoMinSegments || Ls < kAutoMinSegLen)) return sp;
  sp.use = true;
  sp.S = (int)S;
  sp.Ls = (int)Ls;
  sp.nseg = (long)p.N * S;
  return sp;
}

// Workspace of the segmented variant: the segment table [nseg + 1], each sequence's first
// segment [N + 1], then b, M and h_in per (segment, head), each [nseg, H, D, D] fp32.
struct SegLayout {
  size_t cu, first, b, M, h_in, total;
};

SegLayout seg_layout(const gdn::Problem& p, const SegPlan& sp) {
  SegLayout L;
  const size_t ns = (size_t)sp.nseg;
  const size_t st = ns * p.H * (size_t)p.D * p.D * sizeof(float);
  L.cu = 0;
  L.first = align_up((ns + 1) * sizeof(int32_t));
  L.b = L.first + align_up(((size_t)p.N + 1) * sizeof(int32_t));
  L.M = L.b + align_up(st);
  L.h_in = L.M + align_up(st);
  L.total = L.h_in + align_up(st);
  return L;
}

// Stage stop of the fused variant (the page's section 7.4 debugging mode): the fused kernel
// keeps every stage on chip and forms only the chunk-start states h_c and v_new, which its
// store mode writes out.  stop_after = 6 (after chunk_h) is therefore the one stop it
// offers, at its own 64-token chunk (bf16, D = 64 or 128: the store mode's instances).
constexpr int kFusedStop = 6;

bool fused_stop(const gdn_desc* d) {
  return d->variant == GDN_VARIANT_FUSED && d->stop_after != 0;
}

bool fused_stop_ok(const gdn::Problem& p, const gdn_desc* d) {
  return d->stop_after == kFusedStop && gdn::fused_supported(p) && p.D <= 128;
}

// The shape a fused stage stop lays its buffers out for: the fused kernel's chunk.
void fused_stop_chunk(gdn::Problem* p) {
  p->C = kFusedChunk;
  p->max_chunks = (int)(((long long)p->Ttot + kFusedChunk - 1) / kFusedChunk) + p->N;
}

bool seg_ok(const gdn::Problem& p, const gdn_desc* d) {
  return gdn::fused_supported(p) && d->stop_after == 0 &&
         (long long)p.Ttot + p.N <= (1LL << 30);
}

// The staged kernels stage fp32 operands of at most 8192 elements per chunk row block in LDS.
bool staged_ok(const gdn::Problem& p) { return !(p.f32 && p.D * p.C > 8192); }

// The recurrent variant runs one token after another per (sequence, head): AUTO takes it
// when a dense batch has at most kRecurrentMaxT tokens per sequence, or a packed batch at
// most that many on average (decode).  Its grid is N H D / 32 single-wave workgroups.
constexpr int kRecurrentMaxT = 8;

bool recurrent_ok(const gdn::Problem& p, const gdn_desc* d) {
  return d->stop_after == 0 && (long long)p.N * p.H * (p.D / 32) < (1LL << 31);
}

bool recurrent_pays(const gdn::Problem& p, bool dense) {
  return dense ? p.T <= kRecurrentMaxT : (long long)p.Ttot <= (long long)kRecurrentMaxT * p.N;
}

// Variant actually run (after AUTO resolution), or -1 if the request cannot be served.
// `dense`: no cu_seqlens.  `ws`: the workspace the call brings (AUTO picks the segmented
// variant only when it pays off and the workspace is large enough; else the fused one).
int resolve_variant(const gdn_desc* d, const gdn::Problem& p, bool dense, bool ws_check) {
  const bool fused_ok = gdn::fused_supported(p) && d->stop_after == 0;
  switch (d->variant) {
    case GDN_VARIANT_FUSED:
      if (d->stop_after != 0) return fused_stop_ok(p, d) ? GDN_VARIANT_FUSED : -1;
      return fused_ok ? GDN_VARIANT_FUSED : -1;
    case GDN_VARIANT_STAGED: return staged_ok(p) ? GDN_VARIANT_STAGED : -1;
    case GDN_VARIANT_SEGMENTED: return seg_ok(p, d) ? GDN_VARIANT_SEGMENTED : -1;
    case GDN_VARIANT_RECURRENT: return recurrent_ok(p, d) ? GDN_VARIANT_RECURRENT : -1;
    default: {
      if (recurrent_ok(p, d) && recurrent_pays(p, dense)) return GDN_VARIANT_RECURRENT;
      if (!fused_ok) return staged_ok(p) ? GDN_VARIANT_STAGED : -1;
      if (seg_ok(p, d) && seg_plan(p, false, dense).use) {
        if (!ws_check) return GDN_VARIANT_SEGMENTED;
        const size_t need = seg_layout(p, seg_plan(p, false, dense)).total;
        if (d->workspace && d->workspace_bytes >= need && aligned(d->workspace, kAlign))
          return GDN_VARIANT_SEGMENTED;
      }
      return GDN_VARIANT_FUSED;
    }
  }
}

void staged_layout(const gdn::Problem& p, Layout* L) {
  const size_t e = p.f32 ? 4 : 2;            // q/k/v element size
  const size_t eb = p.beta_f32 ? 4 : 2;      // beta element size
  const size_t T = (size_t)p.Ttot, H = (size_t)p.H, D = (size_t)p.D, C = (size_t)p.C;
  const size_t MC = (size_t)p.max_chunks;
  L->bytes[GDN_BUF_CHUNK_TABLE] = MC * 4 * sizeof(int32_t);
  L->bytes[GDN_BUF_SEQ_CHUNKS] = ((size_t)p.N + 1) * sizeof(int32_t);
  L->bytes[GDN_BUF_G_CUM] = T * H * 4;
  L->bytes[GDN_BUF_G_T] = T * H * 4;
  L->bytes[GDN_BUF_BETA_T] = T * H * eb;
  L->bytes[GDN_BUF_A] = T * H * C * 4;
  L->bytes[GDN_BUF_TINV] = T * H * C * e;
  L->bytes[GDN_BUF_W] = T * H * D * e;
  L->bytes[GDN_BUF_U] = T * H * D * e;
  L->bytes[GDN_BUF_H_C] = MC * H * D * D * e;
  L->bytes[GDN_BUF_V_NEW] = T * H * D * e;
  size_t off = 0;
  for (int i = 0; i < GDN_BUF_COUNT; ++i) {
    L->off[i] = off;
    off += align_up(L->bytes[i]);
  }
  L->total = off;
}

// The fused stage stop's buffers: the staged layout at the fused chunk with only the chunk
// table, the sequences' first chunks, h_c and v_new sized (the kernel forms nothing else).
void fused_stop_layout(const gdn::Problem& p, Layout* L) {
  gdn::Problem pc = p;
  fused_stop_chunk(&pc);
  staged_layout(pc, L);
  size_t off = 0;
  for (int i = 0; i < GDN_BUF_COUNT; ++i) {
    const bool kept = i == GDN_BUF_CHUNK_TABLE || i == GDN_BUF_SEQ_CHUNKS ||
                      i == GDN_BUF_H_C || i == GDN_BUF_V_NEW;
    if (!kept) L->bytes[i] = 0;
    L->off[i] = off;
    off += align_up(L->bytes[i]);
  }
  L->total = off;
}

// The fused variant on a packed batch runs its sequences longest first when the workspace
// holds their order (4 bytes per sequence): the order kernel's O(N^2) compares are cheap up
// to this many sequences.  Without it, or beyond, they run in index order (same results).
constexpr int kLptMaxN = 65536;

bool lpt_wanted(const gdn::Problem& p, bool dense) {
  return !dense && p.N > 1 && p.N <= kLptMaxN;
}

size_t lpt_bytes(const gdn::Problem& p) { return align_up((size_t)p.N * sizeof(int32_t)); }

// Workspace of the variant a call resolves to, for one reading of the descriptor.
size_t workspace_for(const gdn_desc* d, const gdn::Problem& p, bool dense) {
  const int v = resolve_variant(d, p, dense, false);
  if (v == GDN_VARIANT_FUSED && fused_stop(d)) {
    Layout L;
    fused_stop_layout(p, &L);
    return L.total;
  }
  if (v == GDN_VARIANT_FUSED) return lpt_wanted(p, dense) ? lpt_bytes(p) : 0;
  if (v == GDN_VARIANT_RECURRENT || v < 0) return 0;
  if (v == GDN_VARIANT_SEGMENTED)
    return seg_layout(p, seg_plan(p, d->variant == GDN_VARIANT_SEGMENTED, dense)).total;
  Layout L;
  staged_layout(p, &L);
  return L.total;
}

// The backward pass recomputes the forward's chunk quantities at C = 64 into the staged
// layout at the front of its workspace, without A (stages 0-2, then T by one launch that
// keeps A on chip, then the chunk-start states and v_new from the fused kernel's store mode
// in bf16, or from stages 5-6 in fp32), then keeps dR
// [Ttot, H, D] and each chunk's end-state gradient [max_chunks, H, D, D] in the q/k/v dtype.
constexpr int kBwdChunk = 64;

struct BwdLayout {
  Layout st;
  size_t dR, dH, order, total;
};

// Shape part of a backward call: the forward's checks with the chunk set to 64 and N as the
// call reads it (cu_seqlens: d->N; else B).
gdn_status bwd_problem(const gdn_desc* d, bool packed, gdn::Problem* p) {
  const gdn_status s = check_desc(d, p);
  if (s != GDN_OK) return s;
  if (packed) {
    if (d->B != 1 || d->N < 0) return GDN_ERR_INVALID_ARG;
    p->N = d->N;
  } else if (d->N != 0 && d->N != d->B) {
    return GDN_ERR_INVALID_ARG;
  }
  p->C = kBwdChunk;
  p->max_chunks = (int)(((long long)p->Ttot + kBwdChunk - 1) / kBwdChunk) + p->N;
  if (!gdn::bwd_supported(*p)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

BwdLayout bwd_layout(const gdn::Problem& p, bool dense) {
  BwdLayout L;
  staged_layout(p, &L.st);
  // A stays on chip (stages 3 and 4 run as one launch), and with the fused recompute (bf16)
  // W and U are never formed: no room for them
  L.st.bytes[GDN_BUF_A] = 0;
  if (gdn::fused_supported(p)) L.st.bytes[GDN_BUF_W] = L.st.bytes[GDN_BUF_U] = 0;
  size_t off = 0;
  for (int i = 0; i < GDN_BUF_COUNT; ++i) {
    L.st.off[i] = off;
    off += align_up(L.st.bytes[i]);
  }
  L.st.total = off;
  const size_t e = p.f32 ? 4 : 2;
  L.dR = L.st.total;
  L.dH = L.dR + align_up((size_t)p.Ttot * p.H * p.D * e);
  // a packed batch's longest-first order, for the two passes over whole sequences
  L.order = L.dH + align_up((size_t)p.max_chunks * p.H * p.D * p.D * e);
  L.total = L.order + (lpt_wanted(p, dense) ? lpt_bytes(p) : 0);
  return L;
}

// Long sequences: the backward's two sequential passes (the recompute of the chunk-start
// states and the reverse pass) run per segment, with the forward's segment plan.  After the
// backward's own buffers: the segment table, the sequences' first segments, then b (reused
// for each segment's own start gradient e), M and h_in (reused for each segment's end
// gradient), as the segmented forward lays them out, and each segment's first chunk
// [nseg + 1].
struct BwdSegLayout {
  SegPlan sp;
  size_t base;  // offset of the segment buffers (the end of BwdLayout)
  SegLayout seg;
  size_t chunks, total;
};

// The plan a backward call runs with: segments only with the fused recompute (bf16), when
// AUTO finds they pay off or GDN_VARIANT_SEGMENTED asks for them; any other variant keeps
// one reverse pass per sequence.
SegPlan bwd_seg_plan(const gdn_desc* d, const gdn::Problem& p, bool dense) {
  if (p.f32 || !gdn::fused_supported(p) || (long long)p.Ttot + p.N > (1LL << 30))
    return SegPlan();
  if (d->variant != GDN_VARIANT_AUTO && d->variant != GDN_VARIANT_SEGMENTED) return SegPlan();
  return seg_plan(p, d->variant == GDN_VARIANT_SEGMENTED, dense);
}

BwdSegLayout bwd_seg_layout(const gdn::Problem& p, const SegPlan& sp, size_t base) {
  BwdSegLayout L;
  L.sp = sp;
  L.base = base;
  L.seg = seg_layout(p, sp);
  L.chunks = base + L.seg.total;
  L.total = L.chunks + align_up(((size_t)sp.nseg + 1) * sizeof(int32_t));
  return L;
}

// Workspace of a backward call for one reading of the descriptor (dense or packed).
size_t bwd_workspace_for(const gdn_desc* d, const gdn::Problem& p, bool dense) {
  const BwdLayout L = bwd_layout(p, dense);
  const SegPlan sp = bwd_seg_plan(d, p, dense);
  return sp.use ? bwd_seg_layout(p, sp, L.total).total : L.total;
}

gdn::Stages stages_at(char* ws, const Layout& L) {
  gdn::Stages st;
  st.table = reinterpret_cast<int32_t*>(ws + L.off[GDN_BUF_CHUNK_TABLE]);
  st.seq_chunks = reinterpret_cast<int32_t*>(ws + L.off[GDN_BUF_SEQ_CHUNKS]);
  st.g_cum = reinterpret_cast<float*>(ws + L.off[GDN_BUF_G_CUM]);
  st.g_t = reinterpret_cast<float*>(ws + L.off[GDN_BUF_G_T]);
  st.beta_t = ws + L.off[GDN_BUF_BETA_T];
  st.A = reinterpret_cast<float*>(ws + L.off[GDN_BUF_A]);
  st.Tinv = ws + L.off[GDN_BUF_TINV];
  st.W = ws + L.off[GDN_BUF_W];
  st.U = ws + L.off[GDN_BUF_U];
  st.h_c = ws + L.off[GDN_BUF_H_C];
  st.v_new = ws + L.off[GDN_BUF_V_NEW];
  return st;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(const gdn_desc* d, gdn_status* status) {
  gdn::Problem p;
  gdn_status s = check_desc(d, &p);
  // the size query cannot see cu_seqlens: N other than 0 or B marks a packed batch, and
  // with B = 1 both readings are possible, so the larger need is reported
  const bool dense = d && (d->N == 0 || d->N == d->B);
  if (s == GDN_OK && resolve_variant(d, p, dense, false) < 0) s = GDN_ERR_UNSUPPORTED;
  if (status) *status = s;
  if (s != GDN_OK) return 0;
  size_t need = workspace_for(d, p, dense);
  if (dense && d->B == 1) {
    gdn::Problem pp = p;
    pp.N = d->N == 0 ? 1 : d->N;
    const size_t packed = workspace_for(d, pp, false);
    if (packed > need) need = packed;
  }
  return need;
}

gdn_status gdn_stage_buffer(const gdn_desc* d, int32_t buf, size_t* offset, size_t* bytes) {
  gdn::Problem p;
  const gdn_status s = check_desc(d, &p);
  if (s != GDN_OK) return s;
  if (buf < 0 || buf >= GDN_BUF_COUNT || !offset || !bytes) return GDN_ERR_INVALID_ARG;
  Layout L;
  if (fused_stop(d)) {
    if (!fused_stop_ok(p, d)) return GDN_ERR_UNSUPPORTED;
    fused_stop_layout(p, &L);
  } else {
    staged_layout(p, &L);
  }
  *offset = L.off[buf];
  *bytes = L.bytes[buf];
  return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* h0,
                         const int32_t* cu_seqlens, float scale, void* o, float* ht,
                         hipStream_t stream) {
  gdn::Problem p;
  gdn_status s = check_desc(d, &p);
  if (s != GDN_OK) return s;
  // an empty token axis needs no token buffers (torch hands out null pointers for them)
  if (p.Ttot > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(g, 4) || !aligned(beta, p.beta_f32 ? 4 : 2) || !aligned(h0, 16) ||
      !aligned(ht, 16) || !aligned(cu_seqlens, 4))
    return GDN_ERR_INVALID_ARG;
  if (cu_seqlens) {
    if (d->B != 1 || d->N < 0) return GDN_ERR_INVALID_ARG;
    p.N = d->N;
    p.max_chunks = (int)(((long long)p.Ttot + p.C - 1) / p.C) + p.N;
  } else if (d->N != 0 && d->N != d->B) {
    return GDN_ERR_INVALID_ARG;
  }
  const int variant = resolve_variant(d, p, cu_seqlens == nullptr, true);
  if (variant < 0) return GDN_ERR_UNSUPPORTED;
  p.scale = scale;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu = cu_seqlens;
  p.o = o;
  p.ht = ht;
  if (p.N == 0) return GDN_OK;

  hipError_t e;
  if (p.Ttot == 0) {
    // no tokens: every sequence is empty and its state passes through (ht = h0, or zeros);
    // the recurrent kernel does exactly that without touching a token buffer
    if (d->stop_after != 0 || !ht) return GDN_OK;
    if ((long long)p.N * p.H * (p.D / 32) >= (1LL << 31)) return GDN_ERR_UNSUPPORTED;
    e = gdn::launch_recurrent(p, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  if (variant == GDN_VARIANT_FUSED && fused_stop(d)) {
    // the chunk table at the fused chunk, then the fused kernel storing h_c and v_new
    Layout L;
    fused_stop_layout(p, &L);
    if (!d->workspace || d->workspace_bytes < L.total || !aligned(d->workspace, kAlign))
      return GDN_ERR_WORKSPACE;
    const gdn::Stages st = stages_at(static_cast<char*>(d->workspace), L);
    gdn::Problem pf = p;
    fused_stop_chunk(&pf);
    e = gdn::launch_chunk_table(pf, st, stream);
    if (e == hipSuccess) {
      pf.o = nullptr;
      pf.ht = nullptr;
      pf.fused_flags = gdn::kFusedNoOutput;
      pf.seq_chunks = st.seq_chunks;
      pf.hc_out = st.h_c;
      pf.vnew_out = st.v_new;
      e = gdn::launch_fused(pf, stream);
    }
  } else if (variant == GDN_VARIANT_FUSED) {
    e = hipSuccess;
    if (lpt_wanted(p, cu_seqlens == nullptr) && d->workspace &&
        d->workspace_bytes >= lpt_bytes(p) && aligned(d->workspace, kAlign)) {
      int32_t* order = static_cast<int32_t*>(d->workspace);
      e = gdn::launch_lpt_order(p.cu, order, p.N, p.T, p.Ttot, stream);
      p.order = order;
    }
    if (e == hipSuccess) e = gdn::launch_fused(p, stream);
  } else if (variant == GDN_VARIANT_RECURRENT) {
    e = gdn::launch_recurrent(p, stream);
  } else if (variant == GDN_VARIANT_SEGMENTED) {
    const bool dense = cu_seqlens == nullptr;
    const SegPlan sp = seg_plan(p, d->variant == GDN_VARIANT_SEGMENTED, dense);
    const SegLayout L = seg_layout(p, sp);
    if (!d->workspace || d->workspace_bytes < L.total || !aligned(d->workspace, kAlign))
      return GDN_ERR_WORKSPACE;
    char* ws = static_cast<char*>(d->workspace);
    int32_t* cu_seg = reinterpret_cast<int32_t*>(ws + L.cu);
    int32_t* seg_first = reinterpret_cast<int32_t*>(ws + L.first);
    float* bm = reinterpret_cast<float*>(ws + L.b);
    float* mm = reinterpret_cast<float*>(ws + L.M);
    float* hin = reinterpret_cast<float*>(ws + L.h_in);
    // every segment is a sequence of a packed batch over the same tokens
    gdn::Problem ps = p;
    ps.N = (int)sp.nseg;
    ps.cu = cu_seg;
    e = dense ? gdn::launch_segment_table(cu_seg, p.N, p.T, sp.S, sp.Ls, stream)
              : gdn::launch_segment_table_packed(p.cu, cu_seg, seg_first, p.N, p.Ttot, sp.Ls,
                                                 (int)sp.nseg, stream);
    // b: each segment from a zero state; M: from the identity with v taken as zero
    if (e == hipSuccess) {
      gdn::Problem pb = ps;
      pb.h0 = nullptr;
      pb.ht = bm;
      pb.fused_flags = gdn::kFusedNoOutput;
      e = gdn::launch_fused(pb, stream);
    }
    if (e == hipSuccess) {
      gdn::Problem pm = ps;
      pm.h0 = nullptr;
      pm.ht = mm;
      pm.fused_flags = gdn::kFusedNoOutput | gdn::kFusedZeroV | gdn::kFusedH0Identity;
      e = gdn::launch_fused(pm, stream);
    }
    // h_in of every segment, and the final state, by composing the maps in order
    if (e == hipSuccess)
      e = gdn::launch_segment_scan_ranges(mm, bm, p.h0, hin, p.ht, dense ? nullptr : seg_first,
                                          p.N, sp.S, p.H, p.D, stream);
    // o of every segment from its true initial state
    if (e == hipSuccess) {
      gdn::Problem po = ps;
      po.h0 = hin;
      po.ht = nullptr;
      e = gdn::launch_fused(po, stream);
    }
  } else {
    Layout L;
    staged_layout(p, &L);
    if (!d->workspace || d->workspace_bytes < L.total || !aligned(d->workspace, kAlign))
      return GDN_ERR_WORKSPACE;
    const gdn::Stages st = stages_at(static_cast<char*>(d->workspace), L);
    e = gdn::launch_staged(p, st, d->stop_after, stream);
  }
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_fused_sigmoid_gating_delta_rule(const gdn_desc* d, const void* q, const void* k,
                                               const void* v, const void* a, const void* b,
                                               const float* A_log, const float* dt_bias,
                                               const float* h0, const int32_t* cu_seqlens,
                                               float scale, void* o, float* ht,
                                               hipStream_t stream) {
  gdn::Problem p;
  gdn_status s = check_desc(d, &p);
  if (s != GDN_OK) return s;
  if (d->variant != GDN_VARIANT_AUTO && d->variant != GDN_VARIANT_RECURRENT)
    return GDN_ERR_UNSUPPORTED;
  if (d->stop_after != 0) return GDN_ERR_INVALID_ARG;
  if (!A_log) return GDN_ERR_INVALID_ARG;
  if (p.Ttot > 0 && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_INVALID_ARG;
  const size_t ab = p.beta_f32 ? 4 : 2;  // a and b share beta's dtype
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(a, ab) || !aligned(b, ab) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(h0, 16) || !aligned(ht, 16) || !aligned(cu_seqlens, 4))
    return GDN_ERR_INVALID_ARG;
  if (cu_seqlens) {
    if (d->B != 1 || d->N < 0) return GDN_ERR_INVALID_ARG;
    p.N = d->N;
  } else if (d->N != 0 && d->N != d->B) {
    return GDN_ERR_INVALID_ARG;
  }
  if (!recurrent_ok(p, d)) return GDN_ERR_UNSUPPORTED;
  p.scale = scale;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = nullptr;
  p.beta = b;
  p.gate_a = a;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.h0 = h0;
  p.cu = cu_seqlens;
  p.o = o;
  p.ht = ht;
  if (p.N == 0) return GDN_OK;
  if (p.Ttot == 0) {
    // no tokens: the states pass through (ht = h0, or zeros), as in gdn_chunk_fwd
    if (!ht) return GDN_OK;
    p.gate_a = nullptr;
  }
  return gdn::launch_recurrent(p, stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_chunk_bwd_workspace_size(const gdn_desc* d, gdn_status* status) {
  gdn::Problem p;
  // N other than 0 or B is read as a packed batch; else the dense reading, whose chunk bound
  // ceil(B T / 64) + B also covers a packed batch of B = 1 and N = 1
  const bool packed = d && d->N != 0 && d->N != d->B;
  gdn_status s = bwd_problem(d, packed, &p);
  if (s == GDN_OK && d->variant == GDN_VARIANT_SEGMENTED && !bwd_seg_plan(d, p, !packed).use)
    s = GDN_ERR_UNSUPPORTED;
  if (status) *status = s;
  if (s != GDN_OK) return 0;
  size_t need = bwd_workspace_for(d, p, !packed);
  if (!packed && d->B == 1) {
    // a single sequence may also come as a packed batch of one (cu_seqlens given)
    gdn::Problem pp = p;
    pp.N = 1;
    const size_t alt = bwd_workspace_for(d, pp, false);
    if (alt > need) need = alt;
  }
  return need;
}

gdn_status gdn_chunk_bwd(const gdn_desc* d, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* h0,
                         const int32_t* cu_seqlens, float scale, const void* dout,
                         const float* dht, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* dh0, hipStream_t stream) {
  gdn::Problem p;
  const gdn_status s = bwd_problem(d, cu_seqlens != nullptr, &p);
  if (s != GDN_OK) return s;
  if (d->grad_dtype != GDN_F32 && d->grad_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->grad_dtype == GDN_BF16 && p.f32) return GDN_ERR_UNSUPPORTED;
  if (p.Ttot > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg ||
                     !dbeta))
    return GDN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(g, 4) || !aligned(beta, p.beta_f32 ? 4 : 2) || !aligned(h0, 16) ||
      !aligned(cu_seqlens, 4) || !aligned(dht, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(dg, 4) || !aligned(dbeta, 4) || !aligned(dh0, 16))
    return GDN_ERR_INVALID_ARG;
  p.scale = scale;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu = cu_seqlens;
  p.o = nullptr;
  p.ht = nullptr;
  if (p.N == 0) return GDN_OK;
  if (p.Ttot == 0) {
    // no tokens: the final state is the initial one, so dh0 = dht (or zeros); the recurrent
    // kernel's pass-through writes exactly that
    if (!dh0) return GDN_OK;
    if ((long long)p.N * p.H * (p.D / 32) >= (1LL << 31)) return GDN_ERR_UNSUPPORTED;
    gdn::Problem pp = p;
    pp.h0 = dht;
    pp.ht = dh0;
    return gdn::launch_recurrent(pp, stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  const bool dense = cu_seqlens == nullptr;
  const BwdLayout L = bwd_layout(p, dense);
  const SegPlan sp = bwd_seg_plan(d, p, dense);
  if (d->variant == GDN_VARIANT_SEGMENTED && !sp.use) return GDN_ERR_UNSUPPORTED;
  const BwdSegLayout SL = bwd_seg_layout(p, sp, L.total);
  const size_t need = sp.use ? SL.total : L.total;
  if (!d->workspace || d->workspace_bytes < need || !aligned(d->workspace, kAlign))
    return GDN_ERR_WORKSPACE;
  char* ws = static_cast<char*>(d->workspace);
  gdn::BwdBuffers b;
  b.st = stages_at(ws, L.st);
  b.dO = dout;
  b.dht = dht;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.grad_bf16 = d->grad_dtype == GDN_BF16;
  b.dg = dg;
  b.dbeta = dbeta;
  b.dh0 = dh0;
  b.dR = ws + L.dR;
  b.dH = ws + L.dH;
  hipError_t e;
  if (sp.use) {
    // stages 0-4, then the segmented forward's maps (b, M) and each segment's true start
    // state h_in, then h_c and v_new from the fused kernel per segment; the reverse pass per
    // segment from a zero end gradient (each segment's own share e), the segments' end
    // gradients composed last to first (dh_in = M^T dh_end + e), and the reverse pass per
    // segment again from its true end gradient, writing dh' and dR
    int32_t* cu_seg = reinterpret_cast<int32_t*>(ws + SL.base + SL.seg.cu);
    int32_t* seg_first = reinterpret_cast<int32_t*>(ws + SL.base + SL.seg.first);
    float* bm = reinterpret_cast<float*>(ws + SL.base + SL.seg.b);
    float* mm = reinterpret_cast<float*>(ws + SL.base + SL.seg.M);
    float* hin = reinterpret_cast<float*>(ws + SL.base + SL.seg.h_in);
    int32_t* seg_chunks = reinterpret_cast<int32_t*>(ws + SL.chunks);
    const int nseg = (int)sp.nseg;
    gdn::Problem ps = p;
    ps.N = nseg;
    ps.cu = cu_seg;
    e = gdn::launch_staged(p, b.st, 4, stream, true);
    if (e == hipSuccess)
      e = dense ? gdn::launch_segment_table(cu_seg, p.N, p.T, sp.S, sp.Ls, stream)
                : gdn::launch_segment_table_packed(p.cu, cu_seg, seg_first, p.N, p.Ttot, sp.Ls,
                                                   nseg, stream);
    if (e == hipSuccess)
      e = gdn::launch_segment_chunks(b.st.seq_chunks, dense ? nullptr : seg_first, seg_chunks,
                                     p.N, sp.S, sp.Ls / kBwdChunk, nseg, stream);
    if (e == hipSuccess) {
      gdn::Problem pb = ps;
      pb.h0 = nullptr;
      pb.ht = bm;
      pb.fused_flags = gdn::kFusedNoOutput;
      e = gdn::launch_fused(pb, stream);
    }
    if (e == hipSuccess) {
      gdn::Problem pm = ps;
      pm.h0 = nullptr;
      pm.ht = mm;
      pm.fused_flags = gdn::kFusedNoOutput | gdn::kFusedZeroV | gdn::kFusedH0Identity;
      e = gdn::launch_fused(pm, stream);
    }
    const int32_t* first = dense ? nullptr : seg_first;
    if (e == hipSuccess)
      e = gdn::launch_segment_scan_ranges(mm, bm, p.h0, hin, nullptr, first, p.N, sp.S, p.H,
                                          p.D, stream);
    if (e == hipSuccess) {
      gdn::Problem pf = ps;
      pf.h0 = hin;
      pf.ht = nullptr;
      pf.fused_flags = gdn::kFusedNoOutput;
      pf.seq_chunks = seg_chunks;
      pf.hc_out = b.st.h_c;
      pf.vnew_out = b.st.v_new;
      e = gdn::launch_fused(pf, stream);
    }
    if (e == hipSuccess)
      e = gdn::launch_bwd_dh(p, b, nseg, seg_chunks, nullptr, nullptr, nullptr, bm, stream);
    if (e == hipSuccess)
      e = gdn::launch_segment_rscan(mm, bm, dht, hin, dh0, first, p.N, sp.S, p.H, p.D, stream);
    if (e == hipSuccess)
      e = gdn::launch_bwd_dh(p, b, nseg, seg_chunks, hin, b.dH, b.dR, nullptr, stream);
    if (e == hipSuccess) e = gdn::launch_bwd_chunk(p, b, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  // a packed batch runs its sequences longest first in the passes over whole sequences
  if (lpt_wanted(p, dense)) {
    int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
    e = gdn::launch_lpt_order(p.cu, order, p.N, p.T, p.Ttot, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
    b.order = order;
  }
  if (gdn::fused_supported(p)) {
    // stages 0-4 (chunk table, Gc, T), then h_c and v_new from the fused kernel
    e = gdn::launch_staged(p, b.st, 4, stream, true);
    if (e == hipSuccess) {
      gdn::Problem pf = p;
      pf.order = b.order;
      pf.fused_flags = gdn::kFusedNoOutput;
      pf.seq_chunks = b.st.seq_chunks;
      pf.hc_out = b.st.h_c;
      pf.vnew_out = b.st.v_new;
      e = gdn::launch_fused(pf, stream);
    }
  } else {
    e = gdn::launch_staged(p, b.st, 6, stream, true);
  }
  if (e == hipSuccess) e = gdn::launch_bwd(p, b, stream);
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_causal_conv1d_fwd(const gdn_conv_desc* d, const void* x, const float* weight,
                                 const float* bias, void* conv_state,
                                 const int32_t* cache_indices,
                                 const int32_t* has_initial_state, const int32_t* cu_seqlens,
                                 void* y, hipStream_t stream) {
  if (!d || !weight) return GDN_ERR_INVALID_ARG;
  if (d->B < 1 || d->T < 0 || d->N < 0 || d->channels < 1 || d->state_lines < 0)
    return GDN_ERR_INVALID_ARG;
  if ((long long)d->B * d->T > 0 && (!x || !y)) return GDN_ERR_INVALID_ARG;
  if (d->dtype != GDN_F32 && d->dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->activation != GDN_ACT_NONE && d->activation != GDN_ACT_SILU) return GDN_ERR_INVALID_ARG;
  if (d->width < 2 || d->width > 4 || d->channels % 8 != 0) return GDN_ERR_UNSUPPORTED;
  const long long Ttot = (long long)d->B * d->T;
  if (Ttot > (1LL << 30) || (long long)d->channels * 8 > (1LL << 30)) return GDN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(conv_state, 16) || !aligned(weight, 4) ||
      !aligned(bias, 4) || !aligned(cache_indices, 4) || !aligned(has_initial_state, 4) ||
      !aligned(cu_seqlens, 4))
    return GDN_ERR_INVALID_ARG;
  if (conv_state && d->state_lines < 1) return GDN_ERR_INVALID_ARG;
  int N = d->N;
  if (cu_seqlens) {
    if (d->B != 1) return GDN_ERR_INVALID_ARG;
  } else {
    if (d->N != 0 && d->N != d->B) return GDN_ERR_INVALID_ARG;
    N = d->B;
  }
  if (N == 0) return GDN_OK;
  gdn::ConvProblem p;
  p.T = d->T;
  p.Ttot = (int)Ttot;
  p.N = N;
  p.C = d->channels;
  p.W = d->width;
  p.lines = conv_state ? d->state_lines : 0;
  p.f32 = d->dtype == GDN_F32;
  p.silu = d->activation == GDN_ACT_SILU;
  p.x = x;
  p.weight = weight;
  p.bias = bias;
  p.state = conv_state;
  p.cache_indices = cache_indices;
  p.has_initial_state = has_initial_state;
  p.cu = cu_seqlens;
  p.y = y;
  return gdn::launch_conv1d(p, stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int32_t gdn_resolved_variant(const gdn_desc* d, const int32_t* cu_seqlens) {
  gdn::Problem p;
  if (check_desc(d, &p) != GDN_OK) return -1;
  if (cu_seqlens) {
    if (d->B != 1 || d->N < 0) return -1;
    p.N = d->N;
  } else if (d->N != 0 && d->N != d->B) {
    return -1;
  }
  return resolve_variant(d, p, cu_seqlens == nullptr, true);
}

int32_t gdn_chunk_bwd_resolved_variant(const gdn_desc* d, const int32_t* cu_seqlens) {
  gdn::Problem p;
  if (bwd_problem(d, cu_seqlens != nullptr, &p) != GDN_OK) return -1;
  const SegPlan sp = bwd_seg_plan(d, p, cu_seqlens == nullptr);
  if (d->variant == GDN_VARIANT_SEGMENTED && !sp.use) return -1;
  if (sp.use) return GDN_VARIANT_SEGMENTED;
  return gdn::fused_supported(p) ? GDN_VARIANT_FUSED : GDN_VARIANT_STAGED;
}

int32_t gdn_resolved_chunk(const gdn_desc* d, const int32_t* cu_seqlens) {
  const int32_t v = gdn_resolved_variant(d, cu_seqlens);
  if (v < 0) return -1;
  if (v == GDN_VARIANT_RECURRENT) return 1;
  if (v == GDN_VARIANT_STAGED) return d->chunk == 0 ? 128 : d->chunk;
  return d->Dk > 128 ? 32 : kFusedChunk;  // the fused kernel's own chunk (also segmented)
}

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape, dtype or variant";
    case GDN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GDN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t gdn_version(void) { return 100; }

}  // extern "C"
