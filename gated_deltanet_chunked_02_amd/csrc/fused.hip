// Fused single-launch chunked Gated DeltaNet forward (the megakernel idea of the
// MegaGDN-PTO page, sections 1.3 and 4.5: all seven stages in one launch, intermediates
// kept on chip), designed for gfx950.
//
// One workgroup owns one (sequence, value head) and walks its chunks in order; nothing
// crosses workgroups, so no grid barrier is needed (the page's all-core SyncAll barrier
// has no counterpart here).  With NJ = 1 (the default) there are D/16 waves, two per SIMD
// at D = 128; wave w owns the 16 state columns 16 w .. 16 w + 15 for all Dk rows, kept as
// fp32 accumulator tiles (NJ = 2: D/32 waves of two 16-column blocks).  Per chunk, with G
// the in-chunk prefix sum of g and h the state at the chunk start:
//
//   A     = (K K^T) * beta_i e^{G_i-G_j}, i > j             (scaled_dot_kkt, section 4.2)
//   R     = diag(beta) (V - diag(e^G) K h)                   (wy_fast + chunk_h, 4.3)
//   (I + A) v_new = R                                        (solve_tril, 4.4, applied)
//   o     = scale (diag(e^G) Q h + (Q K^T * e^{G_i-G_j})_{i>=j} v_new)        (chunk_o)
//   h     = e^{G_last} h + K^T (e^{G_last-G} v_new)          (chunk_h, TileLang page step 1)
//
// (I + A) v_new = R is the same as v_new = U - W h with U = T diag(beta) V, W = T diag(beta
// e^G) K and T = (I + A)^-1, but T is never formed: each wave solves for its own columns
// by blocked forward substitution over the C/16 token blocks.  Every row i of A carries
// beta_i, so with A = diag(beta) A~ the step reads
//
//   v_i = T_ii diag(beta_i) (R_i / beta_i - sum_{j<i} A~_ij v_j),   T_ii = (I + A_ii)^-1,
//
// where the 16 x 16 diagonal inverses come from the nilpotent product
// (I + A_ii)^-1 = (I - A_ii)(I + A_ii^2)(I + A_ii^4)(I + A_ii^8) on the matrix cores, and
// R_i / beta_i = V_i - e^G K_i h needs no beta.  The solve needs no barrier and no
// cross-wave data beyond A.
//
// Two phases and three barriers per chunk:
//   P1  lower tiles of K Q^T and K K^T -> P and -A~ in LDS (packed fp16 16 x 16 tiles; the
//       owner of a diagonal tile replaces it with T_ii diag(beta)); one wave also builds
//       the next chunk's gate vectors.  Barrier.
//   P2  per token block i: K_i h and Q_i h (issued one block ahead), R_i, the substitution
//       step; block i - 1's output products, o store, and (per pair of blocks) the state
//       update h += K^T (e^{G_last-G} v_new) run one block late, independent of block i's
//       chain (K^T fragments by transposing LDS reads).  Barrier; the prefetched K and Q
//       are written to LDS; barrier.
// The next chunk's K, Q and V are loaded into registers during this one (K at its start,
// Q at the start of P2, V half-way through P2, each bounded by the chunk's valid tokens so
// a partial chunk reads zeros); V is written to LDS at the start of the next chunk, which
// reads it only in P2; g and beta are loaded two chunks ahead.  K, Q, V rows are unpadded
// with the 16-byte chunk index XOR-swizzled by the row, which keeps 16-byte fragment reads
// conflict-free.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 16-column state blocks per wave: 2 -> D/32 waves (one per SIMD at D = 128, up to 512
// registers each, every operand fragment feeds two matrix-core instructions); 1 -> D/16
// waves (two per SIMD, 256 registers each, one wave's latency hidden behind the other).
#ifndef GDN_FUSED_NJ
#define GDN_FUSED_NJ 1
#endif
constexpr int kFusedNJ = GDN_FUSED_NJ;
constexpr int kGateWave = 1;  // the wave that builds the gate vectors


template <int D, int C, int NJ_>
struct FusedCfg {
  static constexpr int NJ = NJ_;            // 16-column state blocks per wave
  static constexpr int NW = D / (16 * NJ);  // waves
  static constexpr int NTH = NW * kWave;    // = 4 D / NJ (the launch bound)
  static constexpr int NT = C / 16;         // token blocks per chunk
  static constexpr int NDK = D / 16;        // key blocks
  static constexpr int CPR = D / 8;         // 16-byte pieces per q/k/v row
  static constexpr int TILE = C * D;        // elements of a swizzled [C][D] bf16 tile
  static constexpr int RS = 20;             // row stride (elements) of a packed fp16 tile
  static constexpr int TE = 16 * RS;        // elements per packed 16 x 16 tile
  static constexpr int NLOW = NT * (NT + 1) / 2;
  static constexpr int MAXT = (NT == 2 * NW) ? NT + 1 : (NLOW + NW - 1) / NW;
  static constexpr int RPI = 1024 / (2 * D);        // rows per direct-to-LDS instruction
  static constexpr int NDMA = C / RPI / NW;         // such instructions per wave per tile
  static constexpr int KPL = C * CPR / NTH;         // 16-byte pieces of K per lane
  static constexpr int TPL = C / kWave;             // tokens per lane in the gate scan
  static constexpr int GATES = 2 * 4 * C;           // [2][4][C] G, e^G, beta, e^{G_last-G}
  static_assert(NT % 2 == 0, "token blocks pair up");
  static_assert(NDMA * NW * RPI == C, "tile covered by whole copy instructions");
  static_assert(KPL * NTH == C * CPR, "K tile covered by whole 16-byte loads");
  static_assert((NTH / CPR) % CPR == 0, "row step of the loads is a multiple of the swizzle");
};

// Element offset of (r, k) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int swz(int r, int k) {
  constexpr int CPR = D / 8;
  return r * D + ((((k >> 3) ^ r) & (CPR - 1)) << 3) + (k & 7);
}

// Within a 16-row block (row0 % 16 == 0) the swizzle key of lane l's row is l % 16, so
// the in-row offset of a k chunk depends on the lane only: swz(row0 + l%16, k) =
// row0 * D + swz(l%16, k).
template <int D>
__device__ __forceinline__ int swz_lane(int l, int k) {
  return swz<D>(l & 15, k);
}

// Standard 16-byte fragment (rows row0 + l%16, k0 + 8 (l/16) ...) of a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 frag_swz(const bf16* m, int row0, int k0, int l) {
  return *reinterpret_cast<const bf16x8*>(m + row0 * D + swz_lane<D>(l, k0 + 8 * (l >> 4)));
}

// Key row of the state held in row r (0..15) of key block db.  Row group a = r / 4 of the
// block pair (2p, 2p + 1) covers the eight keys of 16-byte chunk
//   kchunk(p, a) = 2p + a % 2 + (D/16) (a / 2)       (a bijection onto the D/8 chunks),
// block 2p holding the lower four keys for even a and the upper four for odd a (block
// 2p + 1 the others):
//   row r of block db -> key 8 kchunk(db / 2, r / 4) + 4 ((db + r / 4) % 2) + r % 4.
// A 32-deep K h or Q h product then reads each A operand (K or Q row, chunk kchunk(p, g)
// in lane group g) as one contiguous 16-byte fragment, with the B operand built from the
// block pair in the order (2p, 2p + 1) for even g and (2p + 1, 2p) for odd g.  The
// transposing K^T reads of the state update address one group of four keys per lane;
// served 32 lanes (eight token rows) at a time, they are conflict-free when the two key
// groups in the same half of their chunks lie in chunks that differ in bit 3, which the
// row-swizzle then spreads over all 16 chunk positions (D = 128).
template <int D>
__device__ __forceinline__ int kchunk(int p, int a) {
  return 2 * p + (a & 1) + (D / 16) * (a >> 1);
}
template <int D>
__device__ __forceinline__ int state_dk(int db, int r) {
  return 8 * kchunk<D>(db >> 1, r >> 2) + 4 * ((db ^ (r >> 2)) & 1) + (r & 3);
}

// Issue this wave's share of the direct HBM -> LDS copy of one [C][D] tile (rows of one
// head, token stride `stride`), into the swizzled layout.  Rows past `len` re-read the
// last valid row (in bounds); the caller zeroes them once the copy has landed.
template <class F, int D>
__device__ __forceinline__ void dma_tile(bf16* tile, const bf16* src, long stride, int len,
                                         int w, int l) {
  const int slot = l % F::CPR;
#pragma unroll
  for (int j = 0; j < F::NDMA; ++j) {
    const int r0 = (w * F::NDMA + j) * F::RPI;
    const int r = r0 + l / F::CPR;
    const int c = (slot ^ r) & (F::CPR - 1);
    const int rs = min(r, len - 1);
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(src + (long)rs * stride + c * 8),
        (void __attribute__((address_space(3)))*)(tile + r0 * D), 16, 0, 0);
  }
}

// Zero rows [len, C) of a swizzled tile (a partial last chunk).
template <class F, int C>
__device__ __forceinline__ void zero_tail(bf16* tile, int len, int tid) {
  for (int i = tid + len * F::CPR; i < C * F::CPR; i += F::NTH)
    *reinterpret_cast<uint4*>(tile + i * 8) = make_uint4(0, 0, 0, 0);
}

// A raw buffer resource over [base, base + bytes): loads past the end return zero and
// stores past it are dropped (word 3 selects 32-bit raw data on gfx950).  Bounding a
// resource by a chunk's valid tokens makes a partial chunk zero-padded for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// g and beta of a chunk, TPL consecutive tokens per lane (zero past len).  beta is kept
// as raw bits (fp32, or bf16 in the low half) and widened only in chunk_gates, so nothing
// waits for these loads until the chunk's other loads are waited for too.
template <int C>
__device__ __forceinline__ void load_gates(float* ga, uint32_t* be, const float* g,
                                           const void* beta, int beta_f32, int cs, int len,
                                           int h, int H, int l) {
  constexpr int TPL = C / kWave;
  const int bsz = beta_f32 ? 4 : 2;
  const auto rg = buf_rsrc(g + (long)cs * H + h, (uint32_t)(len * H * 4));
  const auto rb = buf_rsrc(static_cast<const char*>(beta) + ((long)cs * H + h) * bsz,
                           (uint32_t)(len * H * bsz));
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    const int t = TPL * l + r;
    ga[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, t * H * 4, 0, 0));
    be[r] = beta_f32 ? __builtin_amdgcn_raw_buffer_load_b32(rb, t * H * 4, 0, 0)
                     : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, t * H * 2, 0, 0);
  }
}

// Wave 0: G = in-chunk prefix sum of g (chunk_cumsum), then G log2(e), e^G, beta and
// e^{G_last - G} (zero past len) into sm[4][C], e^{G_last} into *misc.
template <int C>
__device__ __forceinline__ void chunk_gates(float* sm, float* misc, const float* ga,
                                            const uint32_t* be, int beta_f32, int len, int l) {
  constexpr int TPL = C / kWave;
  float G[TPL];
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < TPL; ++r) s += ga[r];
  const float excl = wave_incl_scan(s) - s;
  float run = excl;
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    run += ga[r];
    G[r] = run;
  }
  const int tl = len - 1;
  float glast = G[0];
#pragma unroll
  for (int r = 1; r < TPL; ++r)
    if ((tl % TPL) == r) glast = G[r];
  glast = __shfl(glast, tl / TPL, kWave);
#pragma unroll
  for (int r = 0; r < TPL; ++r) {
    const int t = TPL * l + r;
    sm[t] = G[r] * 1.4426950408889634f;  // G log2(e): decays are exp2 of differences
    sm[C + t] = __expf(G[r]);
    sm[2 * C + t] = __builtin_bit_cast(float, beta_f32 ? be[r] : be[r] << 16);
    sm[3 * C + t] = t < len ? __expf(glast - G[r]) : 0.f;
  }
  if (l == 0) *misc = __expf(glast);
}

// The u-th lower-triangular 16 x 16 tile (ti >= tj) handled by wave w.  With NT = 2 NW,
// wave w takes block rows w and NT - 1 - w (NT + 1 tiles for every wave); otherwise tiles
// are dealt round-robin in row-major order.  Closed form, so tile loops stay branch-free.
template <int NT, int NW>
__device__ __forceinline__ void lower_tile(int w, int u, int& ti, int& tj) {
  if constexpr (NT == 2 * NW) {
    const bool first = u <= w;
    ti = first ? w : NT - 1 - w;
    tj = first ? u : u - (w + 1);
  } else {
    const int idx = w + NW * u;
    int i = (int)((__builtin_sqrtf(8.f * (float)idx + 1.f) - 1.f) * 0.5f);
    i += ((i + 1) * (i + 2) / 2 <= idx) ? 1 : 0;
    i -= (i * (i + 1) / 2 > idx) ? 1 : 0;
    ti = i;
    tj = idx - i * (i + 1) / 2;
  }
}

// Whether wave w has a u-th tile.
template <int NT, int NW>
__device__ __forceinline__ bool has_tile(int w, int u) {
  constexpr int NLOW = NT * (NT + 1) / 2;
  if constexpr (NT == 2 * NW || NLOW % NW == 0) return true;
  return w + NW * u < NLOW;
}


// Packed lower-triangular storage of 16 x 16 fp16 tiles: tile (ti, tj), tj <= ti, row r,
// column c at tix(ti, tj) + r * RS + c.  RS must be a multiple of 4 (8-byte accesses); of
// 16, 20 and 24, RS = 20 measures fastest on gfx950: it staggers the rows of one 8-byte
// access across the banks, and its 640-byte tile stride puts the two tiles of a paired
// read on opposite halves of the banks.
template <class F>
__device__ __forceinline__ int tix(int ti, int tj) {
  return (ti * (ti + 1) / 2 + tj) * F::TE;
}

__device__ __forceinline__ f32x4 mma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat8h(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mma32h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// One 16-token block through the 32-deep instruction (upper half zero), so that an
// accumulation chain never switches instruction shape between dependent steps.
__device__ __forceinline__ f32x4 mma32h1(f16x4 a, f16x4 b, f32x4 c) {
  const f16x4 z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(cat8h(a, z), cat8h(b, z), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32b(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <typename V4>
__device__ __forceinline__ auto cat8(V4 a, V4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x4 to_h(f32x4 x) { return __builtin_convertvector(x, f16x4); }
__device__ __forceinline__ bf16x4 to_b(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane c
// receives element e = element c % 4 of the 8 bytes that lane 4 e + c / 4 of the group
// addressed.  So if lane c of group g addresses row (R0 + 4 g + c / 4), columns
// (C0 + 4 (c % 4)) .. + 3 of a row-major 16-bit matrix M, lane c receives
// M[R0 + 4 g + e][C0 + c], e = 0..3: a column of M, the k-contiguous operand form of M^T.
template <typename V4>
__device__ __forceinline__ V4 read_tr(const void* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(V4, r);
}

template <int D, int C, int NJ_>
__global__ __launch_bounds__(D * 4 / NJ_) void k_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const void* __restrict__ beta, int beta_f32,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, bf16* __restrict__ o,
    float* __restrict__ ht, int T, int Ttot, int H, int Hg, float scale) {
  typedef FusedCfg<D, C, NJ_> F;
  constexpr int NT = F::NT, NDK = F::NDK, NJ = F::NJ, RS = F::RS, CPR = F::CPR;
  const int n = blockIdx.x / H, h = blockIdx.x - n * H;
  const int hk = h / (H / Hg);
  const long qstride = (long)Hg * D, vstride = (long)H * D;
  const bf16* qh = q + (long)hk * D;
  const bf16* kh = k + (long)hk * D;
  const bf16* vh = v + (long)h * D;

  // Separate LDS objects, so the compiler can tell that reads of K, A and P never touch
  // the Q and V tiles the direct-to-LDS copies are filling, and does not wait for them.
  __shared__ __align__(16) bf16 SK[F::TILE];
  __shared__ __align__(16) bf16 SQ[F::TILE];
  __shared__ __align__(16) bf16 SV[F::TILE];
  __shared__ __align__(16) f16 SA[F::NLOW * F::TE];  // -A below the diagonal, T_ii on it
  __shared__ __align__(16) f16 SP[F::NLOW * F::TE];  // P = (Q K^T * e^{G_i-G_j})_{i>=j}
  __shared__ __align__(16) float sGates[F::GATES];   // [2][4][C]
  __shared__ float sMisc[2];                          // e^{G_last}, double-buffered

  int cs0, L;
  seq_span(cu, n, T, Ttot, cs0, L);
  const int nchunks = (L + C - 1) / C;

  // State: st[j][db] holds rows dk = state_dk<D>(db, 4 (l/16) + e) of column
  // 16 NJ w + NJ (l%16) + j.
  f32x4 st[NJ][NDK];
  const long hoff = ((long)n * H + h) * D * D;
  {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 16 * NJ * w + NJ * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int db = 0; db < NDK; ++db) st[j][db] = zero4();
    if (h0) {
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            st[j][db][e] = h0[hoff + (long)state_dk<D>(db, g4 + e) * D + dv0 + j];
    }
  }
  // bf16 copy of the chunk-start state as the B operands of the K h and Q h products: the
  // pair of key blocks (2p, 2p + 1), swapped in odd lane groups (see state_dk).
  bf16x8 stbo[NJ][NDK / 2];
  auto make_stbo = [&]() {
    const bool odd = (lane_id() >> 4) & 1;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int p = 0; p < NDK / 2; ++p) {
        const bf16x4 lo = to_b(st[j][2 * p]), hi = to_b(st[j][2 * p + 1]);
        stbo[j][p] = odd ? cat8(hi, lo) : cat8(lo, hi);
      }
  };
  make_stbo();

  u32x4 vnext[F::KPL];  // next chunk's V, carried into it
  // g and beta of the next chunk (loaded one chunk earlier) and of the one after it, in
  // the registers of the wave that turns them into gate vectors
  float pg[F::TPL], pg2[F::TPL];
  uint32_t pb[F::TPL], pb2[F::TPL];
  if (nchunks > 0) {
    const int len0 = min(C, L), l = lane_id(), w = wave_id();
    dma_tile<F, D>(SK, kh + (long)cs0 * qstride, qstride, len0, w, l);
    dma_tile<F, D>(SQ, qh + (long)cs0 * qstride, qstride, len0, w, l);
    dma_tile<F, D>(SV, vh + (long)cs0 * vstride, vstride, len0, w, l);
    if (w == kGateWave) {
      load_gates<C>(pg, pb, g, beta, beta_f32, cs0, len0, h, H, l);
      chunk_gates<C>(sGates, sMisc, pg, pb, beta_f32, len0, l);
      if (nchunks > 1)
        load_gates<C>(pg, pb, g, beta, beta_f32, cs0 + C, min(C, L - C), h, H, l);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies have landed
    if (len0 < C) {
      __syncthreads();
      zero_tail<F, C>(SK, len0, threadIdx.x);
      zero_tail<F, C>(SQ, len0, threadIdx.x);
      zero_tail<F, C>(SV, len0, threadIdx.x);
    }
  }
  __syncthreads();

  for (int m = 0; m < nchunks; ++m) {
    const int cs = cs0 + m * C;
    const int len = min(C, L - m * C);
    const int buf = m & 1;
    const float* sG = sGates + buf * 4 * C;
    const float* sEG = sG + C;
    const float* sB = sG + 2 * C;
    const float* sDec = sG + 3 * C;
    // Lane / wave / thread ids are re-derived opaquely at every phase, so the compiler
    // computes each phase's many LDS addresses inside that phase instead of holding them
    // in registers across the chunk.
    int tid, l, w, g4, r16, dvl;
    auto phase = [&]() {
      tid = threadIdx.x;
      opaque(tid);
      l = tid & 63;
      w = __builtin_amdgcn_readfirstlane(tid >> 6);
      g4 = 4 * (l >> 4);
      r16 = l & 15;
      dvl = 16 * NJ * w + NJ * r16;  // this lane's first state column
    };
    phase();

    if (m > 0) {
      // this chunk's V, loaded during the previous one: its tile is not read before the
      // second phase, so it is written here, under the first phase's work
      const uint32_t vr = (uint32_t)tid / CPR, vc = (uint32_t)tid % CPR;
      const int lo = vr * D + (((vc ^ vr) & (CPR - 1)) << 3);
#pragma unroll
      for (int s = 0; s < F::KPL; ++s)
        *reinterpret_cast<u32x4*>(SV + lo + s * (F::NTH / CPR) * D) = vnext[s];
    }
    // Next chunk's K, Q, V into registers, written to LDS once this chunk is done with its
    // tiles.  The loads are spread over the chunk (K now, Q at the start of the second
    // phase, V half-way through it) so the memory pipeline never holds all of them at
    // once.  The gate wave loads g and beta two chunks ahead.
    const bool more = m + 1 < nchunks;
    const int csn = cs + C, lenn = min(C, L - (m + 1) * C);
    u32x4 kp[F::KPL], qp[F::KPL];
    // Lane tid loads rows tid / CPR + s RSTEP (s < KPL), 16-byte piece tid % CPR: a uniform
    // row-block offset plus one per-lane offset.  The resource ends at the chunk's last
    // token, so the rows of a partial chunk past its end load as zero.
    constexpr int RSTEP = F::NTH / CPR;
    const uint32_t rl = (uint32_t)tid / CPR, cl = (uint32_t)tid % CPR;
    auto prefetch = [&](u32x4* dst, const bf16* base, long stride) {
      const auto rs = buf_rsrc(base + (long)csn * stride, (uint32_t)(lenn * stride * 2));
      const int lane = (int)((rl * stride + cl * 8) * 2);
#pragma unroll
      for (int s = 0; s < F::KPL; ++s)
        dst[s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane, (int)(s * RSTEP * stride * 2), 0));
    };
    // the small gate loads (two chunks ahead) first: a wait for them then never waits for
    // the tiles
    if (w == kGateWave && m + 2 < nchunks)
      load_gates<C>(pg2, pb2, g, beta, beta_f32, cs + 2 * C, min(C, L - (m + 2) * C), h, H, l);
    if (more) prefetch(kp, kh, qstride);
    sched_fence();

    // ---- P1: this wave's lower 16 x 16 tiles of K Q^T and K K^T.  Tile (ti, tj) in
    // accumulator form holds, in lane l, row i = 16 ti + l%16 and columns j = 16 tj + 4
    // (l/16) + e: the k-contiguous operand form of that row of P and A.
    // Gate, mask and store one tile (pa = its K Q^T part, aa = its K K^T part): below the
    // diagonal, and on it (masked, and replaced by T_ii).  Gi = G log2(e) of this lane's row
    // and Gj of its four columns are read by the caller ahead of time.
    auto tile_off = [&](int ti, int tj, f32x4 pa, f32x4 aa, float Gi, f32x4 Gj) {
      f32x4 pf, nf;
      f16* at = SA + tix<F>(ti, tj);
      f16* pt = SP + tix<F>(ti, tj);
      // below the diagonal every entry is kept (i > j); beta_i is left to T_ii
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dec = __builtin_amdgcn_exp2f(fminf(Gi - Gj[e], 0.f));
        pf[e] = dec * pa[e];
        nf[e] = -dec * aa[e];
      }
      *reinterpret_cast<f16x4*>(pt + r16 * RS + g4) = to_h(pf);
      *reinterpret_cast<f16x4*>(at + r16 * RS + g4) = to_h(nf);
    };
    auto tile_diag = [&](int ti, int tj, f32x4 pa, f32x4 aa, float Gi, f32x4 Gj) {
      const int i = ti * 16 + r16, j0 = tj * 16 + g4;
      const float nbi = -sB[i];
      const f32x4 bc = *reinterpret_cast<const f32x4*>(sB + j0);
      f32x4 pf, nf;
      f16* at = SA + tix<F>(ti, tj);
      f16* pt = SP + tix<F>(ti, tj);
      // masked entries use a clamped exponent, so they never overflow.  The raw product
      // k_i . k_j of a diagonal tile is symmetric (the same fp32 sum for (i, j) and (j, i)),
      // so each lane also gates it for the mirrored position (row j0 + e, column i): nf
      // holds N^T in accumulator form (N = -A_ii strictly lower) and nfm holds N itself,
      // the two orientations the products below need, without a trip through LDS.
      f32x4 nfm;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dec = __builtin_amdgcn_exp2f(fminf(Gi - Gj[e], 0.f));
        const float decm = __builtin_amdgcn_exp2f(fminf(Gj[e] - Gi, 0.f));
        pf[e] = (i >= j0 + e ? dec : 0.f) * pa[e];
        nf[e] = (i > j0 + e ? nbi * dec : 0.f) * aa[e];
        nfm[e] = (j0 + e > i ? -bc[e] * decm : 0.f) * aa[e];
      }
      *reinterpret_cast<f16x4*>(pt + r16 * RS + g4) = to_h(pf);
      const f16x4 nt = to_h(nf);
      const f16x4 nn = to_h(nfm);
      // T_ii = (I + N + N^2 + ... + N^15) = (I + N)(I + N^2)(I + N^4)(I + N^8).  A product
      // X Y takes X^T and Y in accumulator form, so both orientations of each power are
      // kept; the result is built as T^T, whose accumulator form is the row-major storage
      // of T.
      f32x4 eye;
#pragma unroll
      for (int e = 0; e < 4; ++e) eye[e] = (g4 + e == r16) ? 1.f : 0.f;
      const f32x4 n2 = mma16h(nt, nn, zero4());     // N^2
      const f32x4 n2t = mma16h(nn, nt, zero4());    // (N^2)^T
      const f16x4 h2 = to_h(n2), h2t = to_h(n2t);
      const f32x4 n4 = mma16h(h2t, h2, zero4());    // N^4
      const f32x4 n4t = mma16h(h2, h2t, zero4());   // (N^4)^T
      const f16x4 h4 = to_h(n4), h4t = to_h(n4t);
      const f16x4 h8 = to_h(mma16h(h4t, h4, zero4()));  // N^8
      // Y1 = (I + N^2)^T (I + N)^T = I + N^T + (N^2)^T + (N^2)^T N^T
      const f32x4 y1 = mma16h(h2, nt, eye + nf + n2t);
      const f32x4 y2 = mma16h(h4, to_h(y1), y1);    // (I + (N^4)^T) Y1
      const f32x4 y3 = mma16h(h8, to_h(y2), y2);    // (I + (N^8)^T) Y2 = T_ii^T
      // stored: T_ii diag(beta), i.e. column c of T_ii times beta_c
      *reinterpret_cast<f16x4*>(at + r16 * RS + g4) = to_h(y3 * bc);
    };
    auto tile_out = [&](int ti, int tj, f32x4 pa, f32x4 aa) {
      const float Gi = sG[ti * 16 + r16];
      const f32x4 Gj = *reinterpret_cast<const f32x4*>(sG + tj * 16 + g4);
      if (ti != tj)
        tile_off(ti, tj, pa, aa, Gi, Gj);
      else
        tile_diag(ti, tj, pa, aa, Gi, Gj);
    };
    if constexpr (NT == 2 * F::NW || NT == F::NW) {
      // Block rows pair up as (p, NT - 1 - p), NT + 1 tiles per pair.  With NT = 2 NW wave
      // w owns pair w; with NT = NW waves 2p and 2p + 1 split pair p into 5 and 4 tiles.
      // Each wave walks at most two row segments; a segment's Q and K fragments are loaded
      // once, the products of tile tj + 1 are issued before tile tj's epilogue, and a
      // diagonal tile is always a segment's last.
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        int ti, t0, t1;
        if constexpr (NT == 2 * F::NW) {
          ti = sg == 0 ? w : NT - 1 - w;
          t0 = 0;
          t1 = ti;
        } else {
          const int pp = w >> 1, odd = w & 1;
          const int split = NT / 2 - pp;  // tiles of row NT - 1 - p taken by the even wave
          if (sg == 0) {
            ti = odd ? NT - 1 - pp : pp;
            t0 = odd ? split : 0;
            t1 = ti;
          } else {
            ti = NT - 1 - pp;
            t0 = 0;
            t1 = odd ? -1 : split - 1;  // empty for the odd wave
          }
        }
        if (t1 >= t0) {
          bf16x8 qf[D / 32], kfi[D / 32];
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            qf[kk] = frag_swz<D>(SQ, ti * 16, 32 * kk, l);
            kfi[kk] = frag_swz<D>(SK, ti * 16, 32 * kk, l);
          }
          const float Gi = sG[ti * 16 + r16];
          // a tile's products and its column gates, issued one tile ahead
          auto prods = [&](int tj, f32x4& pa, f32x4& aa, f32x4& Gj) {
            Gj = *reinterpret_cast<const f32x4*>(sG + tj * 16 + g4);
            pa = aa = zero4();
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
              const bf16x8 kf = frag_swz<D>(SK, tj * 16, 32 * kk, l);
              pa = Mma<bf16>::mma(kf, qf[kk], pa);
              aa = Mma<bf16>::mma(kf, kfi[kk], aa);
            }
          };
          f32x4 pa, aa, Gj;
          prods(t0, pa, aa, Gj);
          for (int tj = t0; tj < t1; ++tj) {
            f32x4 pn, an, Gn;
            prods(tj + 1, pn, an, Gn);
            tile_off(ti, tj, pa, aa, Gi, Gj);
            pa = pn;
            aa = an;
            Gj = Gn;
          }
          if (t1 == ti)
            tile_diag(ti, ti, pa, aa, Gi, Gj);
          else
            tile_off(ti, t1, pa, aa, Gi, Gj);
        }
        sched_fence();
      }
    } else {
#pragma unroll
      for (int u = 0; u < F::MAXT; ++u) {
        if (has_tile<NT, F::NW>(w, u)) {
          int ti, tj;
          lower_tile<NT, F::NW>(w, u, ti, tj);
          f32x4 pa = zero4(), aa = zero4();
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const bf16x8 kf = frag_swz<D>(SK, tj * 16, 32 * kk, l);
            pa = Mma<bf16>::mma(kf, frag_swz<D>(SQ, ti * 16, 32 * kk, l), pa);
            aa = Mma<bf16>::mma(kf, frag_swz<D>(SK, ti * 16, 32 * kk, l), aa);
          }
          tile_out(ti, tj, pa, aa);
        }
        sched_fence();
      }
    }
    // The gate wave (an odd wave, one tile fewer than its partner) builds the next
    // chunk's gate vectors in the other buffer, whose last reader was the previous chunk.
    if (w == kGateWave && more)
      chunk_gates<C>(sGates + (buf ^ 1) * 4 * C, sMisc + (buf ^ 1), pg, pb, beta_f32, lenn, l);
    __syncthreads();  // P, -A, T_ii visible

    // ---- P2: per token block i: R_i / beta = V_i - e^G K_i h and Y_i = Q_i h, the forward
    // substitution step, o_i = scale (e^G Y_i + sum_{j<=i} P_ij v_j) and
    // h += K^T (e^{G_last - G} v_new) (two blocks per step).  The K h and Q h products for
    // block i + 1 are issued before block i's dependent chain, and block i's output and
    // update work runs inside block i + 1, so both fill the chain's latency.
    phase();
    if (more) prefetch(qp, qh, qstride);
    sched_fence();
    {
      const float eglast = sMisc[buf];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int db = 0; db < NDK; ++db) st[j][db] *= eglast;
    }
    // Per-lane address parts, fixed for the chunk.  Within a 16-row block the swizzle key
    // of a row depends only on the row's offset in the block, so every LDS access below is
    // one of these lane offsets plus a compile-time block offset, and every output store a
    // uniform block offset plus one of ooff[].
    int voff[4], koff[NDK];
    uint32_t ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      voff[e] = swz<D>(g4 + e, dvl);
      ooff[e] = (uint32_t)(((g4 + e) * H * D + dvl) * 2);
    }
    // one transposing read gives lane (r16, g) its column's V on rows 4g .. 4g + 3 of a
    // token block (one state column per lane)
    const int vtoff = swz<D>(g4 + (r16 >> 2), 16 * w + 4 * (r16 & 3));
#pragma unroll
    for (int db = 0; db < NDK; ++db)
      koff[db] = swz<D>(g4 + (r16 >> 2), state_dk<D>(db, 4 * (r16 & 3)));
    const auto orsrc = buf_rsrc(o + ((long)cs * H + h) * D, (uint32_t)(len * H * D * 2));
    // transposed output layout (one column block per wave): token r16, columns 16 w + 4 g ..
    const uint32_t otoff = (uint32_t)((r16 * H * D + 16 * w + g4) * 2);
    const int oblock = 16 * H * D * 2;  // bytes per 16-token block of o
    const f16* arow = SA + r16 * RS + g4;
    const f16* prow = SP + r16 * RS + g4;
    const f16x4 z4 = {0, 0, 0, 0};

    // v_new of token blocks 2p and 2p + 1 in one fp16 register octet (the B-operand form of
    // a 32-deep product, or with one column block per wave the A-operand form of v_new^T
    // in the output products), zero until written; e^{G_last - G} v_new likewise in bf16.
    f16x8 vp[NT / 2][NJ];
    bf16x8 vbp[NT / 2][NJ];
#pragma unroll
    for (int p2 = 0; p2 < NT / 2; ++p2)
#pragma unroll
      for (int j = 0; j < NJ; ++j) vp[p2][j] = cat8(z4, z4);
    f32x4 xk[NJ], yq[NJ];  // K_i h and Q_i h of the next block
    auto issue_kq = [&](int tb) {
      ARow<bf16, NDK / 2> ak, aq;
#pragma unroll
      for (int p = 0; p < NDK / 2; ++p) {
        // chunk kchunk(p, l / 16) of row tb * 16 + l % 16
        const int ko = tb * 16 * D + swz_lane<D>(l, 8 * kchunk<D>(p, l >> 4));
        ak.f[p] = *reinterpret_cast<const bf16x8*>(SK + ko);
        aq.f[p] = *reinterpret_cast<const bf16x8*>(SQ + ko);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) xk[j] = yq[j] = zero4();
#pragma unroll
      for (int p = 0; p < NDK / 2; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          xk[j] = mma32b(ak.f[p], stbo[j][p], xk[j]);
          // with one column block per wave Y is made transposed (token per lane), like z
          if constexpr (NJ == 1)
            yq[j] = mma32b(stbo[j][p], aq.f[p], yq[j]);
          else
            yq[j] = mma32b(aq.f[p], stbo[j][p], yq[j]);
        }
    };
    // Block i's output and state-update work (z, o, e^{G_last - G} v_i, and the update of
    // the pair (i - 1, i) for odd i).  It runs one block late, inside block i + 1, where it
    // is independent of that block's substitution chain and fills its latency.  It comes
    // before block i + 1's solve in program order, so for even i the pair register of
    // v_i still has a zero upper half.
    auto tail = [&](int i, const f32x4* vn, const f32x4* Yi, f32x4 egs) {
      // o_i = scale (e^G Y_i + sum_{jb <= i} P_{i,jb} v_jb); for even i block i stands
      // alone against a pair register whose upper half is still zero
      f32x4 z[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) z[j] = zero4();
#pragma unroll
      for (int jb = 0; jb + 1 <= i; jb += 2) {
        const f16x8 a = cat8(*reinterpret_cast<const f16x4*>(prow + tix<F>(i, jb)),
                             *reinterpret_cast<const f16x4*>(prow + tix<F>(i, jb + 1)));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          z[j] = NJ == 1 ? mma32h(vp[jb / 2][j], a, z[j]) : mma32h(a, vp[jb / 2][j], z[j]);
      }
      if ((i & 1) == 0) {
        const f16x4 p1 = *reinterpret_cast<const f16x4*>(prow + tix<F>(i, i));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          z[j] = NJ == 1 ? mma32h(vp[i / 2][j], cat8(p1, p1), z[j])
                         : mma32h(cat8(p1, p1), vp[i / 2][j], z[j]);
      }
      // o rows past a partial chunk's end fall outside the output resource and are dropped
      if constexpr (NJ == 1) {
        // z and Y are transposed: lane (r16, g) holds token 16 i + r16, columns
        // 16 w + 4 g .. + 3, stored as one 8-byte word (pairs converted as 32-bit words:
        // this compiler turns an element read of a converted 16-bit vector into a read of
        // element 0)
        const float egt = sEG[i * 16 + r16];
        const f32x2_t o01 = {scale * fmaf(egt, Yi[0][0], z[0][0]), scale * fmaf(egt, Yi[0][1], z[0][1])};
        const f32x2_t o23 = {scale * fmaf(egt, Yi[0][2], z[0][2]), scale * fmaf(egt, Yi[0][3], z[0][3])};
        const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(o01, bf16x2_t));
        const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(o23, bf16x2_t));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 ow = {w01, w23};
        __builtin_amdgcn_raw_buffer_store_b64(ow, orsrc, (int)otoff, i * oblock, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2_t ov;
          ov[0] = (bf16)(scale * fmaf(egs[e], Yi[0][e], z[0][e]));
          ov[1] = (bf16)(scale * fmaf(egs[e], Yi[1][e], z[1][e]));
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, ov), orsrc,
                                                (int)ooff[e], i * oblock, 0);
        }
      }
      {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sDec + i * 16 + g4);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x4 b = to_b(d4 * vn[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) vbp[i / 2][j][4 * (i & 1) + e] = b[e];
        }
      }
      if (i & 1) {
#pragma unroll
        for (int db = 0; db < NDK; ++db) {
          const bf16x8 a = cat8(read_tr<bf16x4>(SK + (i - 1) * 16 * D + koff[db]),
                                read_tr<bf16x4>(SK + i * 16 * D + koff[db]));
#pragma unroll
          for (int j = 0; j < NJ; ++j) st[j][db] = mma32b(a, vbp[i / 2][j], st[j][db]);
        }
      }
    };
    f32x4 vprev[NJ], yprev[NJ], egsprev;
    issue_kq(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      f32x4 acc[NJ], Yi[NJ];
      // e^G of this block's tokens (R and o both use it)
      const f32x4 egs = *reinterpret_cast<const f32x4*>(sEG + i * 16 + g4);
      // R_i / beta = V_i - e^G K_i h (beta is applied by the diagonal solve, T_ii diag(beta))
      if constexpr (NJ == 1) {
        const bf16x4 vv = read_tr<bf16x4>(SV + i * 16 * D + vtoff);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[0][e] = fmaf(-egs[e], xk[0][e], (float)vv[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16* vrow = SV + i * 16 * D + voff[e];
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[j][e] = fmaf(-egs[e], xk[j][e], (float)vrow[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) Yi[j] = yq[j];
      sched_fence();
      if (i + 1 < NT) issue_kq(i + 1);
      if (i == NT / 2 - 1 && more) prefetch(vnext, vh, vstride);
      if (i >= 1) tail(i - 1, vprev, yprev, egsprev);
      // R_i / beta - sum_{jb < i} (A_{i,jb} / beta_i) v_jb in pairs of blocks, the pair
      // holding v_{i-1} last.  For odd i block i - 1 stands alone; its pair register's upper
      // half (v_i) is still zero, so the A operand's upper half only has to be finite.
#pragma unroll
      for (int jb = 0; jb + 1 <= i - 1; jb += 2) {
        const f16x8 a = cat8(*reinterpret_cast<const f16x4*>(arow + tix<F>(i, jb)),
                             *reinterpret_cast<const f16x4*>(arow + tix<F>(i, jb + 1)));
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = mma32h(a, vp[jb / 2][j], acc[j]);
      }
      const f16x4 tf = *reinterpret_cast<const f16x4*>(arow + tix<F>(i, i));
      if (i & 1) {
        const f16x4 a1 = *reinterpret_cast<const f16x4*>(arow + tix<F>(i, i - 1));
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = mma32h(cat8(a1, a1), vp[(i - 1) / 2][j], acc[j]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        vprev[j] = mma16h(tf, to_h(acc[j]), zero4());
        const f16x4 hv = to_h(vprev[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vp[i / 2][j][4 * (i & 1) + e] = hv[e];
        yprev[j] = Yi[j];
      }
      egsprev = egs;
      sched_fence();
    }
    tail(NT - 1, vprev, yprev, egsprev);
    // the next chunk's B operands depend only on this wave's final state
    make_stbo();
    __syncthreads();  // K, Q, V, -A / T_ii and P no longer read
    if (w == kGateWave) {
      // g and beta of the chunk after next move up; done here, long after their loads
      // were issued, because the move waits for them
#pragma unroll
      for (int r = 0; r < F::TPL; ++r) {
        pg[r] = pg2[r];
        pb[r] = pb2[r];
      }
    }
    if (more) {
      // RSTEP is a multiple of the swizzle period, so a lane's swizzle is the same for
      // every s
      const int lo = rl * D + (((cl ^ rl) & (CPR - 1)) << 3);
#pragma unroll
      for (int s = 0; s < F::KPL; ++s) {
        *reinterpret_cast<u32x4*>(SK + lo + s * RSTEP * D) = kp[s];
        *reinterpret_cast<u32x4*>(SQ + lo + s * RSTEP * D) = qp[s];
      }
    }
    __syncthreads();  // next chunk's tiles and gates visible
  }

  if (ht) {
    const int l = lane_id(), w = wave_id();
    const int dv0 = 16 * NJ * w + NJ * (l & 15), g4 = 4 * (l >> 4);
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          ht[hoff + (long)state_dk<D>(db, g4 + e) * D + dv0 + j] = st[j][db][e];
  }
}

template <int D, int C>
hipError_t run_fused(const Problem& p, hipStream_t st) {
  constexpr int NJ = kFusedNJ;
  typedef FusedCfg<D, C, NJ> F;
  const int grid = p.N * p.H;
  if (grid == 0) return hipSuccess;
  k_fused<D, C, NJ><<<grid, F::NTH, 0, st>>>(
      static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), static_cast<const bf16*>(p.v),
      p.g, p.beta, p.beta_f32 ? 1 : 0, p.h0, p.cu, static_cast<bf16*>(p.o), p.ht, p.T, p.Ttot,
      p.H, p.Hg, p.scale);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(const Problem& p) { return !p.f32 && (p.D == 64 || p.D == 128); }

hipError_t launch_fused(const Problem& p, hipStream_t st) {
  if (p.D == 64) return p.C == 64 ? run_fused<64, 64>(p, st) : run_fused<64, 128>(p, st);
  return p.C == 64 ? run_fused<128, 64>(p, st) : run_fused<128, 128>(p, st);
}

}  // namespace gdn
