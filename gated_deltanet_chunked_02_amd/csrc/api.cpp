// C ABI of libgdn (declared in include/gdn.h): host-side validation, the staged
// workspace layout and dispatch to the launchers.  No allocation, no synchronisation.
#include <stdint.h>
#include <string.h>

#include "gdn.h"
#include "gdn_internal.h"

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
  if (d->variant < GDN_VARIANT_AUTO || d->variant > GDN_VARIANT_FUSED) return GDN_ERR_INVALID_ARG;
  if (d->stop_after < 0 || d->stop_after > 6) return GDN_ERR_INVALID_ARG;
  const int C = d->chunk == 0 ? 128 : d->chunk;
  if (C != 64 && C != 128) return GDN_ERR_UNSUPPORTED;
  if (d->Dk != d->Dv) return GDN_ERR_UNSUPPORTED;
  const int D = d->Dk;
  if (D != 64 && D != 128 && D != 256) return GDN_ERR_UNSUPPORTED;
  const bool f32 = d->qkv_dtype == GDN_F32;
  if (f32 && D * C > 8192) return GDN_ERR_UNSUPPORTED;  // fp32 operands: LDS budget
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

// Variant actually run (after AUTO resolution), or -1 if the request cannot be served.
int resolve_variant(const gdn_desc* d, const gdn::Problem& p) {
  const bool fused_ok = gdn::fused_supported(p) && d->stop_after == 0;
  switch (d->variant) {
    case GDN_VARIANT_FUSED: return fused_ok ? GDN_VARIANT_FUSED : -1;
    case GDN_VARIANT_STAGED: return GDN_VARIANT_STAGED;
    default: return fused_ok ? GDN_VARIANT_FUSED : GDN_VARIANT_STAGED;
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

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(const gdn_desc* d, gdn_status* status) {
  gdn::Problem p;
  gdn_status s = check_desc(d, &p);
  if (s == GDN_OK && resolve_variant(d, p) < 0) s = GDN_ERR_UNSUPPORTED;
  if (status) *status = s;
  if (s != GDN_OK) return 0;
  if (resolve_variant(d, p) == GDN_VARIANT_FUSED) return 0;
  Layout L;
  staged_layout(p, &L);
  return L.total;
}

gdn_status gdn_stage_buffer(const gdn_desc* d, int32_t buf, size_t* offset, size_t* bytes) {
  gdn::Problem p;
  const gdn_status s = check_desc(d, &p);
  if (s != GDN_OK) return s;
  if (buf < 0 || buf >= GDN_BUF_COUNT || !offset || !bytes) return GDN_ERR_INVALID_ARG;
  Layout L;
  staged_layout(p, &L);
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
  if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_INVALID_ARG;
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
  const int variant = resolve_variant(d, p);
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
  if (variant == GDN_VARIANT_FUSED) {
    e = gdn::launch_fused(p, stream);
  } else {
    Layout L;
    staged_layout(p, &L);
    if (!d->workspace || d->workspace_bytes < L.total || !aligned(d->workspace, kAlign))
      return GDN_ERR_WORKSPACE;
    char* ws = static_cast<char*>(d->workspace);
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
    e = gdn::launch_staged(p, st, d->stop_after, stream);
  }
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
