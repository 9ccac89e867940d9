// Fused single-launch chunked Gated DeltaNet forward (the megakernel idea of the
// MegaGDN-PTO page, sections 1.3 and 4.5: all seven stages in one launch, intermediates kept
// on chip), designed for gfx950.
//
// One workgroup owns one (sequence, value head) and walks its chunks of CS = 64 tokens in
// order; nothing crosses workgroups.  Wave w owns the 16 state columns 16 w .. 16 w + 15 for
// all Dk rows as fp32 accumulator tiles.  Per chunk, with Gc the prefix sum of g from the
// chunk's start and h the state at the chunk start:
//
//   A     = (K K^T) * beta_i e^{Gc_i-Gc_j}, i > j               (scaled_dot_kkt, section 4.2)
//   R     = diag(beta) (V - diag(e^Gc) K h)                     (wy_fast + chunk_h, 4.3)
//   (I + A) v_new = R                                           (solve_tril, 4.4, applied)
//   o     = scale (diag(e^Gc) Q h + (Q K^T * e^{Gc_i-Gc_j})_{i>=j} v_new)     (chunk_o)
//   h     = e^{Gc_end} h + K^T (e^{Gc_end-Gc} v_new)            (chunk_h, TileLang page step 1)
//
// Every factor is at most 1.  (I + A) v_new = R is the same as v_new = U - W h with
// U = T diag(beta) V, W = T diag(beta e^Gc) K and T = (I + A)^-1, but T is never formed:
// with A = diag(beta) A~, each wave solves for its own columns by forward substitution over
// the chunk's four 16-token blocks,
//
//   v_i = T_ii diag(beta_i) (R_i / beta_i - sum_{j<i} A~_ij v_j),   T_ii = (I + A_ii)^-1,
//
// where the 16 x 16 diagonal inverses come from the nilpotent product
// (I + A_ii)^-1 = (I - A_ii)(I + A_ii^2)(I + A_ii^4)(I + A_ii^8) on the matrix cores.
//
// The matrix-core operands of the substitution and the output (the tiles -A~, T_ii diag(beta)
// and the gated Q K^T, the right-hand sides and v_new) are bf16, whose exponent range is
// fp32's: they hold any magnitude of v and h0 that bf16 inputs can carry.  Only the power
// series of T_ii, whose factors are bounded for keys with beta |k|^2 <= 2 (L2-normalised
// keys), runs in fp16 for its three extra mantissa bits.
//
// The state-independent work of a chunk (its lower 16 x 16 tiles of K K^T and Q K^T, gated
// and masked, the inverses T_ii and the gate vectors) is done one chunk ahead, by waves 0-3
// and one gate wave, while the current chunk is solved; K and Q are therefore triple-buffered in
// LDS: chunk m is being solved, chunk m + 1's tiles are being made, chunk m + 2 is being
// loaded (through registers, with buffer loads bounded at the sequence end, so a partial
// chunk reads zeros).  One barrier per chunk.
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// DK: key dimension (= the value dimension of the tensors); DV: state columns of one
// workgroup (DK / DV workgroups share a (sequence, head)).
template <int DK, int DV>
struct FusedCfg {
  static constexpr int NW = DV / 16;           // waves, one 16-column state block each
  static constexpr int NTH = NW * kWave;       // threads (the launch bound)
  static constexpr int SPLIT = DK / DV;        // workgroups per (sequence, head)
  static constexpr int CS = DK > 128 ? 32 : 64;  // tokens per chunk (LDS holds 3 K/Q tiles)
  static constexpr int NB = CS / 16;           // 16-token blocks per chunk
  static constexpr int NDK = DK / 16;          // key blocks of the state
  static constexpr int CPR = DK / 8;           // 16-byte pieces per q/k row
  static constexpr int CPRV = DV / 8;          // 16-byte pieces per row of this slice of v
  static constexpr int TILE = CS * DK;         // elements of one [CS][DK] q/k tile
  static constexpr int TILEV = CS * DV;        // elements of one [CS][DV] v tile
  static constexpr int KPL = CS * CPR / NTH;   // 16-byte pieces per lane per q/k tile
  static constexpr int RSTEP = NTH / CPR;      // rows between one lane's pieces
  static constexpr int KPLV = CS * CPRV / NTH; // the same for the v tile
  static constexpr int RSTEPV = NTH / CPRV;
  static constexpr int RS = 20;                // row stride of a packed fp16 16 x 16 tile
  static constexpr int TE = 16 * RS;           // elements per packed tile
  static constexpr int NLOW = NB * (NB + 1) / 2;  // lower 16 x 16 tiles of a chunk
  static constexpr int NOFF = 2 * (NLOW - NB);     // off-diagonal tile products (K K^T, Q K^T)
  static_assert(KPL * NTH == CS * CPR && KPLV * NTH == CS * CPRV,
                "tiles covered by whole 16-byte loads");
  static_assert(RSTEP % 16 == 0 && RSTEPV % 16 == 0, "a lane's pieces share one swizzle");
};

// Element offset of (r, k) in a swizzled [rows][D] bf16 tile: the 16-byte piece index is
// XOR-ed with the row's position in its 16-row block, so 16-byte fragment reads of 16 rows
// are conflict-free.
template <int D>
__device__ __forceinline__ int swz(int r, int k) {
  constexpr int CPR = D / 8;
  return r * D + ((((k >> 3) ^ (r & 15)) & (CPR - 1)) << 3) + (k & 7);
}

// Within a 16-row block the swizzle key of lane l's row is l % 16.
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
// block 2p holding the lower four keys for even a and the upper four for odd a.  A 32-deep
// K h or Q h product then reads each A operand (K or Q row, chunk kchunk(p, g) in lane
// group g) as one 16-byte fragment, with the B operand built from the block pair in the
// order (2p, 2p + 1) for even g and (2p + 1, 2p) for odd g; the transposing K^T reads of
// the state update touch both 8-byte halves of the swizzled chunks and so every LDS bank.
// That takes the four chunks of a pair to differ in their low four bits (an LDS bank cycle
// is 16 chunks of 16 bytes): at D = 256 the far chunk is 8 away, not D/16 = 16 (which fell
// on the same banks and made every K^T read a two-way conflict), and pairs p >= 4 take the
// upper 16 chunks, 16 + 2 (p - 4) + a % 2 + 8 (a / 2).
template <int D>
__device__ __forceinline__ int kchunk(int p, int a) {
  if constexpr (D == 256) return 2 * (p & 3) + (a & 1) + 8 * (a >> 1) + 16 * (p >> 2);
  return 2 * p + (a & 1) + (D / 16) * (a >> 1);
}
template <int D>
__device__ __forceinline__ int state_dk(int db, int r) {
  return 8 * kchunk<D>(db >> 1, r >> 2) + 4 * ((db ^ (r >> 2)) & 1) + (r & 3);
}

// A raw buffer resource over [base, base + bytes): loads past the end return zero and
// stores past it are dropped (word 3 selects 32-bit raw data on gfx950).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// An off-diagonal tile product of the side work: rows of block BI, columns of block BJ,
// K K^T (KIND 0) or Q K^T (KIND 1).
template <int BI, int BJ, int KIND>
struct OffTile {
  static constexpr int bi = BI, bj = BJ, kind = KIND;
};

// Packed lower-triangular storage of 16 x 16 fp16 tiles: tile (ti, tj), tj <= ti, row r,
// column c at tix(ti, tj) + r * RS + c.
template <class F>
__device__ __forceinline__ constexpr int tix(int ti, int tj) {
  return (ti * (ti + 1) / 2 + tj) * F::TE;
}

__device__ __forceinline__ f32x4 mma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16b(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
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

// OUT = false: the state-only form (no q read, no Q K^T tiles, no Q h, no o), for the
// segmented variant's passes that only need final states.  STORE = true also writes every
// chunk's start state (bf16, hc[chunk][h][Dk][Dv] with chunk = seq_chunks[n] + m, the
// staged variant's chunk numbering at C = 64) and v_new (bf16, [Ttot][H][Dv]): the
// quantities the backward pass recomputes.
template <int DK, int DV, bool OUT, bool STORE = false>
__global__ __launch_bounds__(DV * 4) void k_fused(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const void* __restrict__ beta, int beta_f32,
    const float* __restrict__ h0, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ order, const int32_t* __restrict__ seq_chunks,
    bf16* __restrict__ hc, bf16* __restrict__ vnew, bf16* __restrict__ o,
    float* __restrict__ ht, int T, int Ttot, int H, int Hg, float scale, int flags) {
  typedef FusedCfg<DK, DV> F;
  constexpr int CS = F::CS, NB = F::NB, NDK = F::NDK, RS = F::RS, TE = F::TE, CPR = F::CPR;
  constexpr int NW = F::NW, CPRV = F::CPRV;
  constexpr int D = DK;  // row length of q, k, v and o
  constexpr float kLog2e = 1.4426950408889634f;
  // XCD-aware order.  The workgroups that read the same q/k rows (the H / Hg value heads of a
  // q/k head, times SPLIT column halves: gsz consecutive indices) should share one XCD's L2,
  // but the hardware deals consecutive workgroups round-robin to the 8 XCDs.  Workgroup p
  // runs on XCD p % 8 at slot p / 8, so it takes member m of group R = (slot / gsz) 8 + XCD:
  // each group's members run on one XCD in consecutive slots, and the groups still start in
  // their global order (a packed batch's longest-first order is kept).  A grid that is not a
  // multiple of 8 gsz keeps the plain order.
  int bid = blockIdx.x;
  {
    const int gsz = F::SPLIT * (H / Hg);
    if (gsz > 1 && gridDim.x % (8 * gsz) == 0) {
      const int xcd = bid & 7, slot = bid >> 3;
      bid = ((slot / gsz) * 8 + xcd) * gsz + slot % gsz;
    }
  }
  const int nh = bid / F::SPLIT, half = bid - nh * F::SPLIT;
  int n = nh / H;  // for a packed batch, a rank that is mapped to a sequence below
  const int h = nh - n * H;
  const int hk = h / (H / Hg);
  const int col0 = half * DV;  // this workgroup's first state column
  const long qstride = (long)Hg * D, vstride = (long)H * D;
  const bf16* qh = q + (long)hk * D;
  const bf16* kh = k + (long)hk * D;
  const bf16* vh = v + (long)h * D + col0;

  __shared__ __align__(16) bf16 SK[3][F::TILE];
  __shared__ __align__(16) bf16 SQ[3][F::TILE];
  __shared__ __align__(16) bf16 SV[2][F::TILEV];
  __shared__ __align__(16) bf16 SA[2][F::NLOW * TE];  // -A~ below the diagonal, T_ii diag(beta) on it
  __shared__ __align__(16) bf16 SP[2][F::NLOW * TE];  // scale (Q K^T * e^{Gc_i-Gc_j})_{i>=j}
  // Gate vectors, made by one wave two chunks ahead (buffer = chunk % 3), per token t:
  __shared__ __align__(16) float SGC[3][CS];  // Gc_t log2(e)
  __shared__ __align__(16) float SBT[3][CS];  // beta_t
  __shared__ __align__(16) float SEF[3][CS];  // e^{Gc_t}
  __shared__ __align__(16) float SEO[3][CS];  // scale e^{Gc_t}
  __shared__ __align__(16) float SDC[3][CS];  // e^{Gc_end - Gc_t}
  __shared__ float SGE[3];                    // e^{Gc_end}

  // Packed batch with a longest-first order (k_lpt_order): workgroup rank n takes the
  // sequence of rank n by length, so the last workgroups to start are the shortest and the
  // batch ends with little imbalance.
  if (order) n = order[n];
  int cs0, L;
  seq_span(cu, n, T, Ttot, cs0, L);
  const int nchunks = (L + CS - 1) / CS;
  // rows of V a chunk reads (none when V is taken as zero)
  auto vlen = [&](int len) { return (flags & kFusedZeroV) ? 0 : len; };

  const int l0 = lane_id(), w0 = __builtin_amdgcn_readfirstlane(wave_id());
  const int r16_0 = l0 & 15, g4_0 = 4 * (l0 >> 4);

  // State: st[db] holds rows dk = state_dk<DK>(db, 4 (l/16) + e) of column
  // col0 + 16 w + l%16.
  f32x4 st[NDK];
  const long hoff = ((long)n * H + h) * D * D;
  {
    const int dv0 = col0 + 16 * w0 + r16_0;
#pragma unroll
    for (int db = 0; db < NDK; ++db) st[db] = zero4();
    if (flags & kFusedH0Identity) {
      // the identity as initial state: the final state is then the chunked map's matrix
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[db][e] = state_dk<DK>(db, g4_0 + e) == dv0 ? 1.f : 0.f;
    } else if (h0) {
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st[db][e] = h0[hoff + (long)state_dk<DK>(db, g4_0 + e) * D + dv0];
    }
  }
  // bf16 copy of the chunk-start state as the B operands of the K h and Q h products: the
  // pair of key blocks (2p, 2p + 1), swapped in odd lane groups (see state_dk).
  bf16x8 stbo[NDK / 2];
  auto make_stbo = [&]() {
    const bool odd = (lane_id() >> 4) & 1;
#pragma unroll
    for (int p = 0; p < NDK / 2; ++p) {
      const bf16x4 lo = to_b(st[2 * p]), hi = to_b(st[2 * p + 1]);
      stbo[p] = odd ? cat8(hi, lo) : cat8(lo, hi);
    }
  };

  // Loads of one staged tile into registers: lane tid holds rows tid / CPR + s RSTEP, piece
  // tid % CPR.  The resource ends at the chunk's last valid token.
  // (q and k tiles: rows of D elements; the v tile: this workgroup's DV columns)
  const uint32_t rl = (uint32_t)threadIdx.x / CPR, cl = (uint32_t)threadIdx.x % CPR;
  const uint32_t rlv = (uint32_t)threadIdx.x / CPRV, clv = (uint32_t)threadIdx.x % CPRV;
  const int lds_lo = swz<D>(rl, cl * 8), lds_lov = swz<DV>(rlv, clv * 8);
  auto load_tile = [&](u32x4* dst, const bf16* base, long stride, int cstart, int clen) {
    const auto rs = buf_rsrc(base + (long)cstart * stride, (uint32_t)(clen * stride * 2));
    const int lane = (int)((rl * stride + cl * 8) * 2);
#pragma unroll
    for (int s = 0; s < F::KPL; ++s)
      dst[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane, (int)(s * F::RSTEP * stride * 2), 0));
  };
  auto store_tile = [&](bf16* tile, const u32x4* src) {
#pragma unroll
    for (int s = 0; s < F::KPL; ++s)
      *reinterpret_cast<u32x4*>(tile + lds_lo + s * F::RSTEP * D) = src[s];
  };
  auto load_vtile = [&](u32x4* dst, int cstart, int clen) {
    // the resource spans the rows' full width; only this workgroup's slice is read
    const auto rs = buf_rsrc(vh + (long)cstart * vstride, (uint32_t)(clen * vstride * 2));
    const int lane = (int)((rlv * vstride + clv * 8) * 2);
#pragma unroll
    for (int s = 0; s < F::KPLV; ++s)
      dst[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane, (int)(s * F::RSTEPV * vstride * 2), 0));
  };
  auto store_vtile = [&](bf16* tile, const u32x4* src) {
#pragma unroll
    for (int s = 0; s < F::KPLV; ++s)
      *reinterpret_cast<u32x4*>(tile + lds_lov + s * F::RSTEPV * DV) = src[s];
  };
  // g and beta of token l (lane l, all CS = 64 tokens of a chunk; zero past the sequence
  // end), loaded by the gate wave, which turns them into the chunk's gate vectors.
  static_assert(CS <= kWave, "one gate per lane");
  constexpr int kGateWave = NW - 1;
  auto load_gate = [&](float& gv, uint32_t& bv, int cstart, int clen) {
    const int bsz = beta_f32 ? 4 : 2;
    const auto rg = buf_rsrc(g + (long)cstart * H + h, (uint32_t)(clen * H * 4));
    const auto rb = buf_rsrc(static_cast<const char*>(beta) + ((long)cstart * H + h) * bsz,
                             (uint32_t)(clen * H * bsz));
    const int t = lane_id();
    gv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, t * H * 4, 0, 0));
    bv = beta_f32 ? __builtin_amdgcn_raw_buffer_load_b32(rb, t * H * 4, 0, 0)
                  : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, t * H * 2, 0, 0);
  };
  // chunk_cumsum and the gate vectors of one chunk into gate buffer gb (gate wave only)
  auto make_gates = [&](int gb, float gv, uint32_t bvr) {
    const int t = lane_id();
    const float Gc = wave_incl_scan(gv) * kLog2e;
    const float gend =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gc), CS - 1));
    const float ef = __builtin_amdgcn_exp2f(Gc);
    if (t < CS) {
      SGC[gb][t] = Gc;
      SBT[gb][t] = __builtin_bit_cast(float, beta_f32 ? bvr : bvr << 16);
      SEF[gb][t] = ef;
      SEO[gb][t] = scale * ef;
      SDC[gb][t] = __builtin_amdgcn_exp2f(gend - Gc);
    }
    if (t == 0) SGE[gb] = __builtin_amdgcn_exp2f(gend);
  };

  // Side work for one chunk (K/Q buffer kb, outputs in buffer ob).  Diagonal block b: the
  // gate vectors of its tokens, T_bb diag(beta) and the masked P_bb.  Below the diagonal:
  // -A~ (no beta: T_ii diag(beta) applies it) and P.  Tile (bi, bj) = K_bj (Q or K)_bi^T in
  // accumulator form holds, in lane l, row i = 16 bi + l%16 and columns j = 16 bj + 4 (l/16)
  // + e: the row-major storage of the tile.
  auto side = [&](int kb, int gb, int ob) {
    const int l = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int r16 = l & 15, g4 = 4 * (l >> 4);
    const bf16* Kx = SK[kb];
    const bf16* Qx = SQ[kb];
    const float* Gc = SGC[gb];
    auto diag = [&](int b) {
      const float Gi = Gc[16 * b + r16], bv = SBT[gb][16 * b + r16];
      const f32x4 Gj = *reinterpret_cast<const f32x4*>(Gc + 16 * b + g4);
      const f32x4 bc = *reinterpret_cast<const f32x4*>(&SBT[gb][16 * b + g4]);
      bf16x8 kf[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) kf[kk] = frag_swz<DK>(Kx, 16 * b, 32 * kk, l);
      f32x4 aa = zero4(), pa = zero4();
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        aa = mma32b(kf[kk], kf[kk], aa);
        if constexpr (OUT) pa = mma32b(kf[kk], frag_swz<DK>(Qx, 16 * b, 32 * kk, l), pa);
      }
      // N = -A_bb strictly lower.  The raw product k_i . k_j is symmetric, so each lane gates
      // it for both orientations: nf holds N^T in accumulator form, nfm holds N.  Masked
      // entries use a clamped exponent, so they never overflow.
      const float nbi = -bv;
      f32x4 nf, nfm, pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = g4 + e;
        const float dec = __builtin_amdgcn_exp2f(fminf(Gi - Gj[e], 0.f));
        const float decm = __builtin_amdgcn_exp2f(fminf(Gj[e] - Gi, 0.f));
        nf[e] = (r16 > j ? nbi * dec : 0.f) * aa[e];
        nfm[e] = (j > r16 ? -bc[e] * decm : 0.f) * aa[e];
        pf[e] = (r16 >= j ? scale * dec : 0.f) * pa[e];
      }
      if constexpr (OUT) *reinterpret_cast<bf16x4*>(&SP[ob][tix<F>(b, b) + r16 * RS + g4]) = to_b(pf);
      const f16x4 nt = to_h(nf), nn = to_h(nfm);
      // T = (I + N)(I + N^2)(I + N^4)(I + N^8): a product X Y takes X^T and Y in
      // accumulator form, so both orientations of each power are kept; T^T is built, whose
      // accumulator form is the row-major storage of T.
      f32x4 eye;
#pragma unroll
      for (int e = 0; e < 4; ++e) eye[e] = (g4 + e == r16) ? 1.f : 0.f;
      const f32x4 n2 = mma16h(nt, nn, zero4());   // N^2
      const f32x4 n2t = mma16h(nn, nt, zero4());  // (N^2)^T
      const f16x4 h2 = to_h(n2), h2t = to_h(n2t);
      const f32x4 n4 = mma16h(h2t, h2, zero4());  // N^4
      const f32x4 n4t = mma16h(h2, h2t, zero4()); // (N^4)^T
      const f16x4 h4 = to_h(n4), h4t = to_h(n4t);
      const f16x4 h8 = to_h(mma16h(h4t, h4, zero4()));  // N^8
      const f32x4 y1 = mma16h(h2, nt, eye + nf + n2t);   // (I + N^2)^T (I + N)^T
      const f32x4 y2 = mma16h(h4, to_h(y1), y1);         // (I + (N^4)^T) Y1
      const f32x4 y3 = mma16h(h8, to_h(y2), y2);         // (I + (N^8)^T) Y2 = T^T
      *reinterpret_cast<bf16x4*>(&SA[ob][tix<F>(b, b) + r16 * RS + g4]) = to_b(y3 * bc);
    };
    // Off-diagonal tile (bi, bj), bj < bi: K K^T -> -A~ (kind 0) or Q K^T -> P (kind 1).
    // Each wave's products are fixed at compile time and all its fragment reads come before
    // its tile stores, so fragments shared by its products are read once.
    auto offdiag = [&](auto... prods) {
      constexpr int NPR = sizeof...(prods);
      constexpr int bi_[NPR] = {decltype(prods)::bi...};
      constexpr int bj_[NPR] = {decltype(prods)::bj...};
      constexpr int kd_[NPR] = {decltype(prods)::kind...};
      f32x4 acc[NPR];
#pragma unroll
      for (int u = 0; u < NPR; ++u) acc[u] = zero4();
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int u = 0; u < NPR; ++u)
          acc[u] = mma32b(frag_swz<DK>(Kx, 16 * bj_[u], 32 * kk, l),
                          frag_swz<DK>(kd_[u] ? Qx : Kx, 16 * bi_[u], 32 * kk, l), acc[u]);
#pragma unroll
      for (int u = 0; u < NPR; ++u) {
        const float Gi = Gc[16 * bi_[u] + r16];
        const f32x4 Gj = *reinterpret_cast<const f32x4*>(Gc + 16 * bj_[u] + g4);
        const float f = kd_[u] ? scale : -1.f;
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = f * __builtin_amdgcn_exp2f(fminf(Gi - Gj[e], 0.f)) * acc[u][e];
        bf16* dst = kd_[u] ? SP[ob] : SA[ob];
        *reinterpret_cast<bf16x4*>(dst + tix<F>(bi_[u], bj_[u]) + r16 * RS + g4) = to_b(x);
      }
    };
    // The twelve products in four shares of three, grouped so that each share reuses
    // operands.  All tile work goes to waves 0 .. NB - 1: each SIMD issues its older wave
    // first, so the younger waves NB .. 2 NB - 1, which only solve (and, for the last one,
    // make the gate vectors), set the pace of the chunk.
    auto offdiag_share = [&](int i) {
      if constexpr (NB == 2) {
        // one off-diagonal tile: K K^T on wave 0, Q K^T on wave 1
        if (i == 0)
          offdiag(OffTile<1, 0, 0>());
        else if (OUT)
          offdiag(OffTile<1, 0, 1>());
        return;
      }
      if constexpr (!OUT) {
        // the K K^T products only
        if (i == 0)
          offdiag(OffTile<1, 0, 0>(), OffTile<2, 0, 0>());
        else if (i == 1)
          offdiag(OffTile<2, 1, 0>(), OffTile<3, 0, 0>());
        else if (i == 2)
          offdiag(OffTile<3, 1, 0>());
        else
          offdiag(OffTile<3, 2, 0>());
        return;
      }
      if (i == 0)
        offdiag(OffTile<1, 0, 0>(), OffTile<1, 0, 1>(), OffTile<2, 0, 0>());
      else if (i == 1)
        offdiag(OffTile<2, 0, 1>(), OffTile<2, 1, 0>(), OffTile<2, 1, 1>());
      else if (i == 2)
        offdiag(OffTile<3, 0, 0>(), OffTile<3, 0, 1>(), OffTile<3, 1, 0>());
      else
        offdiag(OffTile<3, 1, 1>(), OffTile<3, 2, 0>(), OffTile<3, 2, 1>());
    };
    static_assert((NB == 4 && F::NOFF == 12) || (NB == 2 && F::NOFF == 2),
                  "side work dealt evenly");
    static_assert(NW >= NB, "one wave per diagonal block");
    if (w < NB) {
      diag(w);
      offdiag_share(w);
    }
  };

  // Per-lane LDS and output address parts (16-row blocks make every swizzle key a lane
  // constant): V by one transposing read per block (column 16 w + l%16, tokens 4 (l/16)..),
  // K^T of key block db by one transposing read per block, K and Q fragments of pair p.
  const int vtoff = swz<DV>(g4_0 + (r16_0 >> 2), 16 * w0 + 4 * (r16_0 & 3));
  int koff[NDK], kqoff[NDK / 2];
#pragma unroll
  for (int db = 0; db < NDK; ++db)
    koff[db] = swz<DK>(g4_0 + (r16_0 >> 2), state_dk<DK>(db, 4 * (r16_0 & 3)));
#pragma unroll
  for (int p = 0; p < NDK / 2; ++p) kqoff[p] = swz_lane<DK>(l0, 8 * kchunk<DK>(p, l0 >> 4));
  const uint32_t otoff = (uint32_t)((r16_0 * H * D + 16 * w0 + g4_0) * 2);
  const int oblock = 16 * H * D * 2;  // bytes per 16-token block of o

  u32x4 kp[F::KPL], qp[F::KPL], vp[F::KPLV];
  float gvn = 0.f;
  uint32_t bvn = 0;
  if (nchunks > 0) {
    load_tile(kp, kh, qstride, cs0, min(CS, L));
    if constexpr (OUT) load_tile(qp, qh, qstride, cs0, min(CS, L));
    load_vtile(vp, cs0, vlen(min(CS, L)));
    if (w0 == kGateWave) {
      load_gate(gvn, bvn, cs0, min(CS, L));
      make_gates(0, gvn, bvn);
      if (nchunks > 1) {
        load_gate(gvn, bvn, cs0 + CS, min(CS, L - CS));
        make_gates(1, gvn, bvn);
      }
    }
    store_tile(SK[0], kp);
    if constexpr (OUT) store_tile(SQ[0], qp);
    store_vtile(SV[0], vp);
    if (nchunks > 1) {
      load_tile(kp, kh, qstride, cs0 + CS, min(CS, L - CS));
      if constexpr (OUT) load_tile(qp, qh, qstride, cs0 + CS, min(CS, L - CS));
      store_tile(SK[1], kp);
      if constexpr (OUT) store_tile(SQ[1], qp);
    }
    __syncthreads();
    side(0, 0, 0);
    make_stbo();
    __syncthreads();
  }

  // the loop body with compile-time buffer indices (kb = m % 3, tb = m % 2)
  auto body = [&](int m, auto kbt, auto tbt) {
    constexpr int kb = decltype(kbt)::value, tb = decltype(tbt)::value;
    constexpr int kb1 = kb == 2 ? 0 : kb + 1, kb2 = kb1 == 2 ? 0 : kb1 + 1;
    const int cs = cs0 + m * CS;
    const int len = min(CS, L - m * CS);
    const bool more1 = m + 1 < nchunks, more2 = m + 2 < nchunks;
    // the next chunk's side work first, then the loads of later chunks, so the side work
    // does not hold registers with loads in flight
    if (more1) side(kb1, kb1, tb ^ 1);
    sched_fence();
    if (more2) {
      const int c2 = cs + 2 * CS, len2 = min(CS, L - (m + 2) * CS);
      if (w0 == kGateWave) load_gate(gvn, bvn, c2, len2);
      load_tile(kp, kh, qstride, c2, len2);
      if constexpr (OUT) load_tile(qp, qh, qstride, c2, len2);
    }
    if (more1) load_vtile(vp, cs + CS, vlen(min(CS, L - (m + 1) * CS)));
    sched_fence();

    const int l = lane_id();
    const int r16 = l & 15, g4 = 4 * (l >> 4);
    const bf16* Kc = SK[kb];
    const bf16* Qc = SQ[kb];
    const bf16* vt = SV[tb] + vtoff;
    const bf16* Ac = SA[tb] + r16 * RS + g4;
    const bf16* Pc = SP[tb] + r16 * RS + g4;
    const float* efp = SEF[kb] + g4;
    const float* eop = SEO[kb] + r16;
    const float* dcp = SDC[kb] + g4;
    const auto orsrc = buf_rsrc(o + ((long)cs * H + h) * D + col0,
                                (flags & kFusedNoOutput) ? 0u : (uint32_t)(len * H * D * 2));
    if constexpr (STORE) {
      // the chunk-start state, for the backward
      const long cb = ((long)(seq_chunks[n] + m) * H + h) * D * D;
      const int dv0 = col0 + 16 * w0 + r16;
#pragma unroll
      for (int db = 0; db < NDK; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hc[cb + (long)state_dk<DK>(db, g4 + e) * D + dv0] = (bf16)st[db][e];
    }

    // K h and Q h of every block with the chunk-start state; Y = Q h is made transposed
    // (token per lane), like the output product below
    f32x4 xk[NB], yq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      xk[b] = yq[b] = zero4();
      if constexpr (DK > 128) {
        // 256 keys: the K fragments, then the Q fragments, so that only one set is live
        bf16x8 f[NDK / 2];
#pragma unroll
        for (int p = 0; p < NDK / 2; ++p)
          f[p] = *reinterpret_cast<const bf16x8*>(Kc + kqoff[p] + b * 16 * D);
#pragma unroll
        for (int p = 0; p < NDK / 2; ++p) xk[b] = mma32b(f[p], stbo[p], xk[b]);
        if constexpr (OUT) {
          sched_fence();
#pragma unroll
          for (int p = 0; p < NDK / 2; ++p)
            f[p] = *reinterpret_cast<const bf16x8*>(Qc + kqoff[p] + b * 16 * D);
#pragma unroll
          for (int p = 0; p < NDK / 2; ++p) yq[b] = mma32b(stbo[p], f[p], yq[b]);
        }
      } else {
        bf16x8 kf[NDK / 2], qf[NDK / 2];
#pragma unroll
        for (int p = 0; p < NDK / 2; ++p) {
          kf[p] = *reinterpret_cast<const bf16x8*>(Kc + kqoff[p] + b * 16 * D);
          if constexpr (OUT) qf[p] = *reinterpret_cast<const bf16x8*>(Qc + kqoff[p] + b * 16 * D);
        }
#pragma unroll
        for (int p = 0; p < NDK / 2; ++p) xk[b] = mma32b(kf[p], stbo[p], xk[b]);
        if constexpr (OUT) {
#pragma unroll
          for (int p = 0; p < NDK / 2; ++p) yq[b] = mma32b(stbo[p], qf[p], yq[b]);
        }
      }
    }
    // forward substitution, outputs and the update operands, block by block.  The tiles
    // and v_new enter the matrix cores as bf16, whose exponent range is fp32's: any magnitude
    // of v and h0 that bf16 holds stays representable (and each value keeps its own
    // exponent, so large and small values side by side keep their relative precision).
    bf16x4 vnb[NB], vb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // R / beta - sum_{j<b} A~_bj v_j = V - e^Gc (K h) + sum_{j<b} (-A~_bj) v_j: lane
      // (l%16, g) holds tokens 4 g + e of column 16 w + l%16
      const bf16x4 vv = read_tr<bf16x4>(vt + b * 16 * DV);
      const f32x4 ef = *reinterpret_cast<const f32x4*>(efp + 16 * b);
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(-ef[e], xk[b][e], (float)vv[e]);
#pragma unroll
      for (int j = 0; j < b; ++j)
        acc = mma16b(*reinterpret_cast<const bf16x4*>(Ac + tix<F>(b, j)), vnb[j], acc);
      // v_b = T_bb diag(beta) (...)
      const f32x4 vn =
          mma16b(*reinterpret_cast<const bf16x4*>(Ac + tix<F>(b, b)), to_b(acc), zero4());
      vnb[b] = to_b(vn);
      if constexpr (STORE) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * b + g4 + e;
          if (t < len) vnew[((long)(cs + t) * H + h) * D + col0 + 16 * w0 + r16] = (bf16)vn[e];
        }
      }
      // o^T = scale e^Gc Y^T + sum_{j<=b} v_j^T (scale P_bj)^T: lane (l%16, g) holds token
      // 16 b + l%16, columns 16 w + 4 g .. + 3, stored as one 8-byte word (pairs converted
      // as 32-bit words: this compiler turns an element read of a converted 16-bit vector
      // into a read of element 0)
      if constexpr (OUT) {
        f32x4 z = zero4();
#pragma unroll
        for (int j = 0; j <= b; ++j)
          z = mma16b(vnb[j], *reinterpret_cast<const bf16x4*>(Pc + tix<F>(b, j)), z);
        const float egt = eop[16 * b];
        const f32x2_t o01 = {fmaf(egt, yq[b][0], z[0]), fmaf(egt, yq[b][1], z[1])};
        const f32x2_t o23 = {fmaf(egt, yq[b][2], z[2]), fmaf(egt, yq[b][3], z[3])};
        const u32x2 ow = {__builtin_bit_cast(uint32_t, __builtin_convertvector(o01, bf16x2_t)),
                          __builtin_bit_cast(uint32_t, __builtin_convertvector(o23, bf16x2_t))};
        __builtin_amdgcn_raw_buffer_store_b64(ow, orsrc, (int)otoff, b * oblock, 0);
      }
      // e^{Gc_end - Gc} v_new, the update operand
      const f32x4 dc = *reinterpret_cast<const f32x4*>(dcp + 16 * b);
      vb[b] = to_b(dc * vn);
    }
    // h = e^{Gc_end} h + K^T (e^{Gc_end-Gc} v_new), two blocks per 32-deep product (K^T
    // fragments by transposing LDS reads)
    {
      const float ge = SGE[kb];
#pragma unroll
      for (int db = 0; db < NDK; ++db) st[db] *= ge;
#pragma unroll
      for (int pb = 0; pb < NB / 2; ++pb) {
        const bf16x8 vv8 = cat8(vb[2 * pb], vb[2 * pb + 1]);
#pragma unroll
        for (int db = 0; db < NDK; ++db) {
          const bf16x8 a = cat8(read_tr<bf16x4>(Kc + koff[db] + 2 * pb * 16 * D),
                                read_tr<bf16x4>(Kc + koff[db] + (2 * pb + 1) * 16 * D));
          st[db] = mma32b(a, vv8, st[db]);
        }
      }
    }
    make_stbo();
    if (more2) {
      store_tile(SK[kb2], kp);
      if constexpr (OUT) store_tile(SQ[kb2], qp);
      if (w0 == kGateWave) make_gates(kb2, gvn, bvn);
    }
    if (more1) store_vtile(SV[tb ^ 1], vp);
    __syncthreads();
  };
  for (int m = 0; m < nchunks; m += 6) {
    body(m, std::integral_constant<int, 0>(), std::integral_constant<int, 0>());
    if (m + 1 < nchunks) body(m + 1, std::integral_constant<int, 1>(), std::integral_constant<int, 1>());
    if (m + 2 < nchunks) body(m + 2, std::integral_constant<int, 2>(), std::integral_constant<int, 0>());
    if (m + 3 < nchunks) body(m + 3, std::integral_constant<int, 0>(), std::integral_constant<int, 1>());
    if (m + 4 < nchunks) body(m + 4, std::integral_constant<int, 1>(), std::integral_constant<int, 0>());
    if (m + 5 < nchunks) body(m + 5, std::integral_constant<int, 2>(), std::integral_constant<int, 1>());
  }

  if (ht) {
    const int dv0 = col0 + 16 * w0 + r16_0;
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ht[hoff + (long)state_dk<DK>(db, g4_0 + e) * D + dv0] = st[db][e];
  }
}

template <int DK, int DV, bool OUT, bool STORE = false>
hipError_t run_fused(const Problem& p, hipStream_t st) {
  const int grid = p.N * p.H * FusedCfg<DK, DV>::SPLIT;
  if (grid == 0) return hipSuccess;
  k_fused<DK, DV, OUT, STORE><<<grid, FusedCfg<DK, DV>::NTH, 0, st>>>(
      static_cast<const bf16*>(p.q), static_cast<const bf16*>(p.k), static_cast<const bf16*>(p.v),
      p.g, p.beta, p.beta_f32 ? 1 : 0, p.h0, p.cu, p.cu ? p.order : nullptr, p.seq_chunks,
      static_cast<bf16*>(p.hc_out), static_cast<bf16*>(p.vnew_out), static_cast<bf16*>(p.o),
      p.ht, p.T, p.Ttot, p.H, p.Hg, p.scale, p.fused_flags);
  return hipGetLastError();
}

// Longest-processing-time-first order of a packed batch: order[rank] = m, where the rank of
// sequence m counts the sequences longer than m, and those of equal length before it.  One
// thread per sequence, the lengths staged through LDS in blocks; O(N^2) compares over the
// whole grid (about 10 us at N = 4096), and the ranks are a permutation.
__global__ __launch_bounds__(256) void k_lpt_order(const int32_t* __restrict__ cu,
                                                   int32_t* __restrict__ order, int N, int T,
                                                   int Ttot) {
  __shared__ int lens[1024];
  const int m = blockIdx.x * 256 + threadIdx.x;
  int lm = 0;
  if (m < N) {
    int s0;
    seq_span(cu, m, T, Ttot, s0, lm);
  }
  int r = 0;
  for (int j0 = 0; j0 < N; j0 += 1024) {
    const int nj = min(1024, N - j0);
    __syncthreads();
    for (int i = threadIdx.x; i < nj; i += 256) {
      int s0, l0;
      seq_span(cu, j0 + i, T, Ttot, s0, l0);
      lens[i] = l0;
    }
    __syncthreads();
    for (int i = 0; i < nj; ++i) {
      const int lj = lens[i];
      r += (lj > lm) || (lj == lm && j0 + i < m);
    }
  }
  if (m < N) order[r] = m;
}

}  // namespace

hipError_t launch_lpt_order(const int32_t* cu, int32_t* order, int N, int T, int Ttot,
                            hipStream_t st) {
  if (N <= 0) return hipSuccess;
  k_lpt_order<<<(N + 255) / 256, 256, 0, st>>>(cu, order, N, T, Ttot);
  return hipGetLastError();
}

bool fused_supported(const Problem& p) {
  return !p.f32 && (p.D == 64 || p.D == 128 || p.D == 256);
}

hipError_t launch_fused(const Problem& p, hipStream_t st) {
  if (p.hc_out) {
    // the backward's recompute: state-only, storing the chunk-start states and v_new
    if (p.D == 64) return run_fused<64, 64, false, true>(p, st);
    if (p.D == 128) return run_fused<128, 128, false, true>(p, st);
    return hipErrorInvalidValue;
  }
  // D = 256: two workgroups per (sequence, head), 128 state columns each
  if (p.fused_flags & kFusedNoOutput) {
    if (p.D == 64) return run_fused<64, 64, false>(p, st);
    if (p.D == 128) return run_fused<128, 128, false>(p, st);
    return run_fused<256, 128, false>(p, st);
  }
  if (p.D == 64) return run_fused<64, 64, true>(p, st);
  if (p.D == 128) return run_fused<128, 128, true>(p, st);
  return run_fused<256, 128, true>(p, st);
}

}  // namespace gdn
