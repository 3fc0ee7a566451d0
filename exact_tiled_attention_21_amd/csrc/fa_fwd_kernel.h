// Exact attention forward kernel (FlashAttention-2 work partitioning) for gfx950.
//
// Parallel over (query tile, head, batch): the "Flash attention gpu" page
// notes that batch and heads are independent and that different query blocks
// are independent too, so each workgroup owns 128 query rows of one head and
// loops over all key/value tiles ("flash-attention-v100" README: FlashAttention-2
// reworked the parallelism and work partitioning). Four waves of 32 rows each;
// the Q fragment stays in VGPRs for the whole loop; K/V tiles are staged
// through a double-buffered, XOR-swizzled LDS ring; the online softmax keeps a
// running max and sum per row and rescales the O accumulator, so the Nq x Nk
// scores never leave registers.
//
// K/V tiles move from HBM to LDS by DMA (buffer loads that write LDS
// directly: no staging registers, no LDS store instructions); the swizzle is
// applied by the choice of global chunk each lane fetches, and rows past the
// end of the keys read as zero through the buffer bounds check.
//
// Per loop step j: issue the DMA of tile j+1 into the stage freed by step
// j-1; S_j = K_j Q^T on MFMA; softmax; O += V_j P_j on MFMA; barrier. Each
// tile's loads have a whole step to land. The kernel is held to 256 registers
// or fewer (a few spilled at d = 256), so two workgroups (four at d = 32,
// three at d = 64, 96 and 128) share a CU and each SIMD can interleave one
// wave's exponentials with another wave's matrix products. Long fp16
// sequences at d = 128 without a band use one wide workgroup per CU instead:
// eight waves, 256 rows, two waves per SIMD (see FwdCfg).
//
// The reference max m used in P = exp2(s * scale * log2(e) - m) need not be
// the running max: O and the row sum share it, so the result is the same for
// any m as long as P stays in range. Masked tiles take the tile's row max and
// move m when it grows by more than 2^kLazy (at d = 256 they follow the
// unmasked scheme below, which needs fewer registers). Unmasked tiles skip the
// row max altogether: they form P against the current m and take the (rare)
// max-and-rebase path only when some lane's sum of the tile's probabilities
// exceeds kSumCap, which bounds every P of the tile, or when m is not set yet.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, bool BAND, bool WIDE = false> struct FwdCfg {
  // four waves, one per SIMD, and two or more workgroups per CU (several waves
  // per SIMD, each workgroup with its own barrier): a second (third, fourth) wave
  // overlaps one wave's softmax with another's products. Registers allow four
  // at d = 32, three at d = 64 and two up to d = 192 without spills; d = 256 at
  // two spills a few dozen bytes per lane and is still much faster than at one.
  // d = 96 and 128 take 32-key tiles, which free the registers (and LDS) for a
  // third wave (with a band only without the per-wave skip of masked tiles,
  // which would make it spill).
  // WIDE (d = 128 fp16 without a band, long sequences): one workgroup of eight
  // waves per CU, two per SIMD, 256 rows sharing each 64-key K/V tile, so each
  // K/V byte crosses from L2 into LDS half as often per query row as with
  // three 128-row workgroups.
  static_assert(!WIDE || (D == 128 && !BAND), "the wide shape is d = 128 without a band");
  static constexpr bool kNarrow = (D == 96 || D == 128) && !WIDE;
  static constexpr int WPE = (D <= 32) ? 4 : (D <= 64 || kNarrow) ? 3 : 2;
  static constexpr int NW = WIDE ? 8 : 4;            // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BR = 32 * NW;                 // query rows per workgroup
  static constexpr int BC = (D <= 128 && !kNarrow) ? 64 : 32;    // keys per LDS tile
  static constexpr int KB = BC / 32;                 // 32-key blocks of S^T
  static constexpr int NS = D / 16;                  // 16-wide d slices (QK^T depth)
  static constexpr int NCB = D / 32;                 // 32-wide d blocks of O^T
  static constexpr int NT = BC / 16;                 // 16-key slices (PV depth)
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int NPIECE = TILE_BYTES / 1024;           // 1 KB DMA pieces per tile
  static constexpr int NDMA = (NPIECE + NW - 1) / NW;        // pieces per wave (the last may idle)
  static constexpr bool EVEN = NPIECE % NW == 0;
  static_assert(BR == fwd_rows(D, WIDE), "rows per workgroup");
  static_assert(TILE_BYTES % 1024 == 0, "tile must split into whole DMA pieces");
};

constexpr float kLazy = 8.0f;      // a tile's max moves m when it exceeds m by this (log2 units)
constexpr float kSumCap = 16384.f;  // larger per-lane tile sums of P redo the tile after a rebase

// The sequence one workgroup works on: its query and key counts, the first
// rows of its Q/O and K/V in the (padded or packed) tensors, and the index of
// its first LSE entry.
struct FwdSeq {
  int nq, nk;
  size_t q_row0, k_row0, lse0;
};

// LDS of one workgroup: two stages each for K and V, as separate objects so the
// compiler knows a DMA into one stage never feeds a read of the other.
template <int D, bool BAND, bool WIDE = false> struct FwdLds {
  static constexpr int TB = FwdCfg<D, BAND, WIDE>::TILE_BYTES;
  char* k[2];
  char* v[2];
};

// Per-wave state and the steps of the tile loop (device code only).
template <int D, bool BF16, bool BAND, bool WIDE = false> struct FwdWave {
  using C = FwdCfg<D, BAND, WIDE>;
  using E = Elem<BF16>;
  static constexpr bool kBand = BAND;
  using T = typename E::T;
  using V8 = typename E::V8;
  typedef V8 PF[C::NT];
  typedef f32x16 SA[C::KB];

  const FwdArgs& a;
  const FwdSeq& sq;
  int lane, wave, hh, ln32;
  int qrow, q0w, diag;
  // tiles [jlo, jhi) hold a key some row of the workgroup sees; tiles
  // [jua, jub) need no element mask for any row (the others are computed with it)
  int jlo, jhi, jua, jub;
  int lo_key, hi_key;   // keys this lane's row sees: lo_key <= key <= hi_key
  int w_lo, w_hi;       // keys some row of this wave sees (w_lo > w_hi: none), wave-uniform
  float sl2;
  V8 qf[C::NS];
  f32x16 oacc[C::NCB];
  // running reference max (log2 units); per-lane partial row sums of the rounded
  // probabilities (O's normaliser) and, for bf16, of the unrounded ones (the LSE's)
  float m_run, l_part, l_exact;
  // DMA
  const char* kg;
  const char* vg;
  uint32_t rowbytes;
  int64_t valid;
  uint32_t goff[C::NDMA];
  // LDS read offsets of this lane's fragments: K slice s, V^T c-block cb (low and high 4 keys)
  // (d = 256: recomputed per read from the bases below instead; the 32 registers
  // they would take are what two waves per SIMD need)
  static constexpr bool kPreOfs = D <= 192;
  uint32_t kofs[C::NS], vlo[C::NCB], vhi[C::NCB];
  uint32_t kro, kxo, vb0, vb1, vx0, vx1;

  // first key row i sees, and one past its last (band and cache bounds)
  __device__ __forceinline__ int lbound(int i) const {
    return (BAND && a.wl >= 0) ? max(0, i + diag - a.wl) : 0;
  }
  __device__ __forceinline__ int rbound(int i) const {
    return (BAND && a.wr >= 0) ? min(sq.nk, i + diag + a.wr + 1) : sq.nk;
  }

  __device__ __forceinline__ FwdWave(const FwdArgs& args, const FwdSeq& seq, int g, int qt)
      : a(args), sq(seq) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    hh = lane >> 5;
    ln32 = lane & 31;
    sl2 = a.sl2;
    rowbytes = static_cast<uint32_t>(a.Hkv) * D * 2;
    offsets();
    begin(g, qt);
  }

  // The state of one query tile (rows of tile qt of sequence sq, KV head g):
  // key extents, tile ranges, K/V sources, and cleared accumulators.
  __device__ __forceinline__ void begin(int g, int qt) {
    q0w = qt * C::BR + wave * 32;
    qrow = q0w + ln32;
    diag = sq.nk - sq.nq;

    // Key extents. Row i sees keys j with i + diag - wl <= j <= i + diag + wr
    // (the band of a sliding window; causal is wl = none, wr = 0), clipped to
    // [0, nk). The first row has the smallest bounds, the last the largest.
    const int nk = sq.nk;
    const bool has_l = BAND && a.wl >= 0, has_r = BAND && a.wr >= 0;
    const int q0 = qt * C::BR;
    const int last_wg = min(q0 + C::BR, sq.nq) - 1;
    lo_key = has_l ? qrow + diag - a.wl : -0x7fffffff;
    hi_key = min(nk, has_r ? qrow + diag + a.wr + 1 : nk) - 1;
    // the wave's first row has the smallest bounds, its last valid row the largest
    const int w_last = min(q0w + 31, sq.nq - 1);
    w_lo = has_l ? max(0, q0w + diag - a.wl) : 0;
    w_hi = min(nk, has_r ? w_last + diag + a.wr + 1 : nk) - 1;
    if (w_last < q0w) w_hi = -1;   // the wave has no rows
    // tiles of the workgroup
    const int kb = lbound(q0), ke = rbound(last_wg);
    jlo = kb / C::BC;
    jhi = ke > kb ? (ke + C::BC - 1) / C::BC : jlo;
    // tiles without element masks: inside every row's band and below nk
    jua = max(jlo, has_l ? (lbound(last_wg) + C::BC - 1) / C::BC : 0);
    jub = min(jhi, min(nk / C::BC, has_r ? max(0, rbound(q0)) / C::BC : nk / C::BC));
    if (q0 + C::BR > sq.nq) jub = jua;   // a wave of this workgroup has no rows
    if (jub < jua) jub = jua;

    // HBM -> LDS by DMA through buffer resources (rows >= Nk read as 0)
    kg = kv_base(a.k, g);
    vg = kv_base(a.v, g);
    valid = static_cast<int64_t>(sq.nk - 1) * rowbytes + D * 2;

#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] = f32x16{};
    m_run = kNegInf;
    l_part = 0.f;
    l_exact = 0.f;
  }

  // first K (or V) row of KV head g of the sequence
  __device__ __forceinline__ const char* kv_base(const void* base, int g) const {
    return reinterpret_cast<const char*>(base) + (sq.k_row0 * a.Hkv + g) * D * 2;
  }

  // Offsets that depend on the lane only. DMA piece i of this wave fills LDS bytes
  // [(i * NW + wave) * 1024, +1024): lane l writes 16 bytes at +16 l, i.e.
  // physical chunk pch of row r, so it fetches logical chunk pch ^ swz(r) of that row.
  __device__ __forceinline__ void offsets() {
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
      const uint32_t p = (i * C::NW + wave) * 1024 + lane * 16;
      const uint32_t r = p / (D * 2), pch = (p % (D * 2)) / 16;
      goff[i] = r * rowbytes + ((pch ^ Swz<D>::f(r)) << 4);
    }

    // LDS read offsets (the swizzle only sees the low 4 row bits), computed once:
    // one register each saves an ALU op per fragment read in the loop
    // K: row 32kb + ln32, chunk (2s | hh) ^ swz(ln32) -> byte (kxo ^ 32s) + row offset
    kro = ln32 * (D * 2);
    kxo = (static_cast<uint32_t>(hh) ^ Swz<D>::f(ln32)) << 4;
    // V: rows 16t + vrow0 (+8), chunk (4cb + vxl) ^ swz(row) -> byte (vx ^ 64cb) + row offset
    const uint32_t vj = lane & 15, vcb = (lane >> 4) & 1;
    const uint32_t vrow0 = 4 * hh + (vj >> 2), vrow1 = vrow0 + 8;
    const uint32_t vxl = 2 * vcb + ((vj & 3) >> 1);
    vx0 = (vxl ^ Swz<D>::f(vrow0)) << 4;
    vx1 = (vxl ^ Swz<D>::f(vrow1)) << 4;
    vb0 = vrow0 * (D * 2) + 8 * (vj & 1);
    vb1 = vrow1 * (D * 2) + 8 * (vj & 1);
#pragma unroll
    for (int i = 0; i < C::NS; ++i) kofs[i] = (kxo ^ (32u * i)) + kro;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) {
      vlo[cb] = (vx0 ^ (64u * cb)) + vb0;
      vhi[cb] = (vx1 ^ (64u * cb)) + vb1;
    }
  }

  // Q fragment (B operand): Q[qrow][16s + 8hh .. +7], sign-flipped for a negative
  // scale. All loads are issued before the flip, which waits for them once.
  __device__ __forceinline__ void load_q(int hq) {
    fetch_q(qf, sq, qrow, hq);
    flip_q(qf);
  }
  __device__ __forceinline__ void fetch_q(V8 (&dst)[C::NS], const FwdSeq& s_, int row, int hq) const {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((s_.q_row0 + row) * a.Hq + hq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) dst[s] = row < s_.nq ? *reinterpret_cast<const V8*>(qp + 16 * s) : V8{};
  }
  __device__ __forceinline__ void flip_q(V8 (&f)[C::NS]) const {
    if (a.negate_q) {
#pragma unroll
      for (int s = 0; s < C::NS; ++s) f[s] = -f[s];
    }
  }

  __device__ __forceinline__ void dma(const char* base, int tile, char* lds) const {
    const int64_t off = static_cast<int64_t>(tile) * C::BC * rowbytes;
    const int64_t rem = valid - off;
    const uint32_t nrec = rem > 0 ? static_cast<uint32_t>(rem > 0x7fffffff ? 0x7fffffff : rem) : 0u;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base + (rem > 0 ? off : 0)), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i)
      if (C::EVEN || i * C::NW + wave < C::NPIECE)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + (i * C::NW + wave) * 1024), 16, goff[i], 0, 0, 0);
  }

  // LDS fragments: K (A operand of S^T) and V^T (A operand of O^T) at precomputed offsets
  __device__ __forceinline__ V8 kfrag(const char* kt, int kb, int s) const {
    const uint32_t off = kb * 32 * (D * 2) + (kPreOfs ? kofs[s] : (kxo ^ (32u * s)) + kro);
    return lds_read_v8<V8>(kt, off);
  }
  __device__ __forceinline__ V8 vfrag(const char* vt, int cb, int t) const {
    const uint32_t lo = t * 16 * (D * 2) + (kPreOfs ? vlo[cb] : (vx0 ^ (64u * cb)) + vb0);
    const uint32_t hi = t * 16 * (D * 2) + (kPreOfs ? vhi[cb] : (vx1 ^ (64u * cb)) + vb1);
    return __builtin_bit_cast(V8, __builtin_shufflevector(lds_read_tr(vt, lo), lds_read_tr(vt, hi),
                                                          0, 1, 2, 3, 4, 5, 6, 7));
  }

  // S_j = K_j Q^T (K fragments from LDS, Q from registers). K fragments are read
  // kPre MFMAs ahead through a small rolling buffer; the order is pinned for the
  // scheduler, which would otherwise issue each read right before its MFMA.
  static constexpr int kQkMf = C::KB * C::NS;            // MFMAs in S_j
  static constexpr int kPre = kQkMf < 4 ? kQkMf : 4;     // K fragments in flight
  __device__ __forceinline__ void qk(const char* kt, SA& sacc) const {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) sacc[kb] = f32x16{};
    V8 kf[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) kf[i] = kfrag(kt, i % C::KB, i / C::KB);
#pragma unroll
    for (int i = 0; i < kQkMf; ++i) {
      sacc[i % C::KB] = E::mfma(kf[i % kPre], qf[i / C::KB], sacc[i % C::KB]);
      if (i + kPre < kQkMf) kf[i % kPre] = kfrag(kt, (i + kPre) % C::KB, (i + kPre) / C::KB);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int i = 0; i < kQkMf; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kPre < kQkMf) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }

  // scores of keys this lane's row does not see -> -inf (tile jt)
  __device__ __forceinline__ void mask(SA& sacc, int jt) const {
    const int k0 = jt * C::BC;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key < lo_key || key > hi_key) sacc[kb][r] = kNegInf;
      }
  }
  // mask (if asked) and row max of the raw scores of tile jt
  template <bool MASK>
  __device__ __forceinline__ float rowmax(SA& sacc, int jt) const {
    if (MASK) mask(sacc, jt);
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    return halves_max(mx);
  }
  // move the reference max if the tile's max exceeds it by more than 2^kLazy
  // (rare after the first tiles), rescaling O and the row sum
  __device__ __forceinline__ void rebase(float mx) {
    const float mxs = (mx == kNegInf) ? kNegInf : mx * sl2;
    const bool need = mxs > m_run + kLazy;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      const float m_new = need ? mxs : m_run;
      // 1 when this row keeps its reference (also for a row still at -inf), 0 when it had none
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);
      l_part *= alpha;
      if (BF16) l_exact *= alpha;
#pragma unroll
      for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] *= alpha;
      m_run = m_new;
    }
  }
  // probabilities of a tile against the reference max, as MFMA B operands rounded
  // to the element type. O is normalised by the sum of the rounded values, so its
  // weights are the rounded probabilities divided by their own total and a
  // dominant key carries no rounding error into O. fp16: that sum is formed here
  // (two values per v_dot2, fp32 accumulate), is within 2^-11 of the unrounded one
  // and also serves the LSE. bf16: the unrounded fp32 values are summed here for
  // the LSE (the rounded sum can be 2^-9 off) and the rounded sum is formed by
  // rounded_sum() once the P V products are issued. Either return value bounds
  // every probability of the tile.
  template <bool MASK>
  __device__ __forceinline__ float probs(const SA& sacc, PF& pf) const {
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      f32x16 tmp;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sv = sacc[t >> 1][8 * (t & 1) + i];
        float p = exp2_fast(__builtin_fmaf(sv, sl2, -m_use));
        if (MASK) p = (sv == kNegInf) ? 0.f : p;
        if (BF16) ps[i & 3] += p;
        tmp[i] = p;
      }
      pf[t] = to_v8<BF16>(tmp, 0);
      if (!BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ps[i & 1] = dot2_ones<BF16>(pf[t], i, ps[i & 1]);
      }
    }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  }
  // this lane's sum of the rounded probabilities of a tile (bf16)
  __device__ __forceinline__ float rounded_sum(const PF& pf) const {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < C::NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[i] = dot2_ones<BF16>(pf[t], i, rs[i]);
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  }
  // adds a tile's sums: `ps` from probs(), the rounded sum (bf16) after the P V products
  __device__ __forceinline__ void add_sum(float ps) {
    if (BF16) l_exact += ps;
    else l_part += ps;
  }

  // O += V_j P_j, with the transposing reads of V kVPre MFMAs ahead through a
  // rolling buffer (slot i % (kVPre + 1) is refilled right after MFMA i used it)
  static constexpr int kPvMf = C::NT * C::NCB;
  static constexpr int kVPre = 1;
  __device__ __forceinline__ void pv(const char* vt, const PF& pf) {
    constexpr int NB = kVPre + 1;
    V8 vf[NB];
#pragma unroll
    for (int i = 0; i < NB && i < kPvMf; ++i) vf[i] = vfrag(vt, i % C::NCB, i / C::NCB);
#pragma unroll
    for (int i = 0; i < kPvMf; ++i) {
      oacc[i % C::NCB] = E::mfma(vf[i % NB], pf[i / C::NCB], oacc[i % C::NCB]);
      if (i + NB < kPvMf) vf[i % NB] = vfrag(vt, (i + NB) % C::NCB, (i + NB) / C::NCB);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NB, 0);
#pragma unroll
    for (int i = 0; i < kPvMf; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + NB < kPvMf) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }

  // One step over tile j (stage ST); the DMA started here fills tile j+1 into
  // stage ST^1, which was last read in step j-1. TAIL steps cover the tiles
  // where some wave of the workgroup needs an element mask (key tail, causal
  // diagonal) or has no visible key; the other steps are straight-line code so
  // the O accumulators keep their registers across the loop.
  template <int ST, bool TAIL>
  __device__ __forceinline__ void step(int j, const FwdLds<D, BAND, WIDE>& lds) {
    if (!kPreOfs) asm volatile("" : "+v"(kxo), "+v"(vx0), "+v"(vx1));
    if (j + 1 < jhi) {
      dma(kg, j + 1, lds.k[ST ^ 1]);
      dma(vg, j + 1, lds.v[ST ^ 1]);
    }
    if (!TAIL) {
      SA sacc;
      PF pf;
      qk(lds.k[ST], sacc);
      // no row max: redo the tile after a rebase only if a probability may be
      // out of range (or m is not set yet); a NaN sum also takes that path
      float ps = probs<false>(sacc, pf);
      const bool need = !(ps <= kSumCap) || m_run == kNegInf;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
        rebase(rowmax<false>(sacc, j));
        ps = probs<false>(sacc, pf);
      }
      add_sum(ps);
      pv(lds.v[ST], pf);
      if (BF16) l_part += rounded_sum(pf);
    } else {
      // masked tiles (diagonal, band edges, key tail) with the element mask; a
      // wave none of whose rows sees a key of the tile skips the products (all
      // its probabilities would be 0) but still takes part in the DMA and
      // barrier. Only below d = 96: the branch costs ~45 registers, which at
      // d = 96 and 128 would block the third wave and beyond would spill.
      if (D >= 96 || (j * C::BC <= w_hi && (j + 1) * C::BC - 1 >= w_lo && w_lo <= w_hi)) {
        SA sacc;
        PF pf;
        qk(lds.k[ST], sacc);
        if constexpr (D > 192) {
          // the unmasked tiles' scheme on the masked scores: no row max unless a
          // sum passes the cap or the reference is not set yet (fewer registers
          // live at once: the d = 256 kernels spill less)
          mask(sacc, j);
          float ps = probs<true>(sacc, pf);
          const bool need = !(ps <= kSumCap) || m_run == kNegInf;
          if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
            rebase(rowmax<false>(sacc, j));
            ps = probs<true>(sacc, pf);
          }
          add_sum(ps);
        } else {
          rebase(rowmax<true>(sacc, j));
          add_sum(probs<true>(sacc, pf));
        }
        pv(lds.v[ST], pf);
        if (BF16) l_part += rounded_sum(pf);
      }
    }
    __syncthreads();
  }

  // O = O / l, LSE = m + log(l); rows with no visible key give 0 and -inf.
  // The accumulator gives each lane 4-element pieces of its row, so storing it
  // directly writes 16 scattered bytes per row and instruction; instead the
  // wave's 32 x D tile of O goes through its own slice of the (now idle) K/V
  // LDS stages, and each 16-byte store instruction then writes whole rows.
  __device__ __forceinline__ void finish(int hq, const FwdLds<D, BAND, WIDE>& lds) {
    constexpr int WPS = C::BC / 32;                // waves per LDS stage
    const int st = wave / WPS;
    finish_via(hq, (st == 0 ? lds.k[0] : st == 1 ? lds.k[1] : st == 2 ? lds.v[0] : lds.v[1]) +
                       (wave % WPS) * (32 * D * 2));
  }
  // the same through the wave's own [32][D] slice `ot` of some LDS buffer
  __device__ __forceinline__ void finish_via(int hq, char* const ot) {
    const float l = halves_sum(l_part);
    const float l_lse = BF16 ? halves_sum(l_exact) : l;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // this wave's tile: [32][D] of the element type, 16-byte chunks swizzled by row
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        // columns 32cb + 8gr + 4hh .. +3 of row ln32: half hh of chunk 4cb + gr
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (T)(oacc[cb][4 * gr + e] * inv);
        *reinterpret_cast<T4*>(ot + Swz<D>::off(ln32, 4 * cb + gr) + 8 * hh) = w;
      }
    wave_lds_sync();
    // chunk c = 64 i + lane of the tile: row c / (D / 8), 16-byte chunk c % (D / 8)
    constexpr int CPR = D / 8;
    T* const obase = reinterpret_cast<T*>(a.o) + (sq.q_row0 * a.Hq + hq) * D;
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
      const uint32_t c = 64 * i + lane;
      const uint32_t row = c / CPR, x = c % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ot + Swz<D>::off(row, x));
      const int r = q0w + static_cast<int>(row);
      if (r < sq.nq) *reinterpret_cast<u32x4*>(obase + static_cast<size_t>(r) * a.Hq * D + 8 * x) = v;
    }
    if (a.lse != nullptr && hh == 0 && qrow < sq.nq)
      a.lse[sq.lse0 + qrow] =
          l_lse > 0.f ? (m_run + __log2f(l_lse)) * kLn2 : kNegInf;
  }
};

// The tile loop of one query tile: masked tiles before the unmasked run (the
// left edge of a band; all of them when there is no unmasked run), the unmasked
// run two tiles per iteration with compile-time stages, then the masked tiles
// after it (key tail, diagonal, right edge of a band). Tile j lives in stage
// (j - jlo) & 1.
template <class W, class L>
__device__ __forceinline__ void fwd_tiles(W& w, const L& lds) {
  int j = w.jlo;
  // masked tiles before the unmasked run (the left edge of a band); all of
  // them when there is no unmasked run. Without a band the unmasked run starts
  // at the first tile, and the masked tiles after it are all there is otherwise.
  if constexpr (W::kBand) {
    const int head_end = w.jub > w.jua ? w.jua : w.jhi;
    for (; j + 2 <= head_end; j += 2) {   // j - jlo is even here
      w.template step<0, true>(j, lds);
      w.template step<1, true>(j + 1, lds);
    }
    if (j < head_end) {
      w.template step<0, true>(j, lds);
      ++j;
    }
  }
  // the unmasked run, two tiles per iteration with compile-time stages
  if (j < w.jub && ((j - w.jlo) & 1)) {
    w.template step<1, false>(j, lds);
    ++j;
  }
  for (; j + 2 <= w.jub; j += 2) {
    w.template step<0, false>(j, lds);
    w.template step<1, false>(j + 1, lds);
  }
  // masked tiles after it (key tail, diagonal, right edge of a band)
  if (j < w.jhi && ((j - w.jlo) & 1)) {
    w.template step<1, true>(j, lds);
    ++j;
  }
  for (; j + 2 <= w.jhi; j += 2) {
    w.template step<0, true>(j, lds);
    w.template step<1, true>(j + 1, lds);
  }
  if (j < w.jhi) w.template step<0, true>(j, lds);
}

template <int D, bool BF16, bool BAND, bool WIDE = false>
__global__ __launch_bounds__((FwdCfg<D, BAND, WIDE>::THREADS))
__attribute__((amdgpu_waves_per_eu((FwdCfg<D, BAND, WIDE>::WPE), (FwdCfg<D, BAND, WIDE>::WPE)))) void fa_fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<D, BAND, WIDE>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[C::TILE_BYTES];

  // workgroup -> (query tile, head, batch)
  int qt, hb;
  if (BAND) {
    // with a causal band the last query tiles see the most keys
    int o;
    blocked_order(blockIdx.x, a.n_qtiles, a.Hq * a.B, a.hb, o, hb, a.group);
    qt = a.n_qtiles - 1 - o;
  } else {
    xcd_heads(blockIdx.x, a.n_qtiles, a.Hq * a.B, gridDim.x, qt, hb, a.group);
  }
  const int hq = hb % a.Hq;
  const int b = hb / a.Hq;
  const int g = hq / a.group;

  // the sequence: a padded batch element, or one packed sequence whose bounds
  // come from the prefix sums (clamped into the tensors, so a malformed table
  // cannot lead outside them); workgroups past its last query row have nothing to do
  FwdSeq sq;
  if (a.cu_q != nullptr) {
    const int q_lo = min(max(a.cu_q[b], 0), a.total_q);
    const int q_hi = min(max(a.cu_q[b + 1], q_lo), a.total_q);
    const int k_lo = min(max(a.cu_k[b], 0), a.total_k);
    const int k_hi = min(max(a.cu_k[b + 1], k_lo), a.total_k);
    sq = FwdSeq{q_hi - q_lo, k_hi - k_lo, static_cast<size_t>(q_lo), static_cast<size_t>(k_lo),
                static_cast<size_t>(hq) * a.total_q + q_lo};
    if (qt * C::BR >= sq.nq) return;   // uniform over the workgroup, before any barrier
  } else {
    sq = FwdSeq{a.Nq, a.Nk, static_cast<size_t>(b) * a.Nq, static_cast<size_t>(b) * a.Nk,
                (static_cast<size_t>(b) * a.Hq + hq) * a.Nq};
  }

  FwdWave<D, BF16, BAND, WIDE> w(a, sq, g, qt);
  const FwdLds<D, BAND, WIDE> lds{{k_lds0, k_lds1}, {v_lds0, v_lds1}};
  // tile j lives in stage (j - jlo) & 1; the first tile's DMA goes out before
  // the Q loads, so the prologue waits for one memory latency, not two
  if (w.jhi > w.jlo) {
    w.dma(w.kg, w.jlo, lds.k[0]);
    w.dma(w.vg, w.jlo, lds.v[0]);
  }
  w.load_q(hq);
  __syncthreads();
  fwd_tiles(w, lds);
  w.finish(hq, lds);
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, bool bf16, bool band, hipStream_t stream) {
  using C = FwdCfg<D, false>;   // threads per workgroup: the same with and without a band
  static_assert(C::THREADS == FwdCfg<D, true>::THREADS, "one block size");
  const dim3 grid(static_cast<unsigned>(a.n_qtiles) * a.Hq * a.B);
  const dim3 block(C::THREADS);
  (void)hipGetLastError();   // start from a clean error state
  if constexpr (D == 128) {
    if (a.wide && !bf16 && !band) {   // n_qtiles then counts 256-row tiles
      fa_fwd_kernel<D, false, false, true><<<grid, dim3(FwdCfg<D, false, true>::THREADS), 0, stream>>>(a);
      return hipGetLastError();
    }
  }
  if (bf16) {
    if (band) fa_fwd_kernel<D, true, true><<<grid, block, 0, stream>>>(a);
    else fa_fwd_kernel<D, true, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (band) fa_fwd_kernel<D, false, true><<<grid, block, 0, stream>>>(a);
    else fa_fwd_kernel<D, false, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fa
