// Exact attention backward pass on gfx950 (MFMA 32x32x16).
//
// For O = softmax(scale Q K^T) V (with a causal mask or sliding-window band, if
// any) and an upstream
// gradient dO, with P the softmax probabilities and D_i = sum_c dO[i][c] O[i][c]:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// As in the forward pass no score matrix is stored: P is recomputed tile by tile
// from the forward's log-sum-exp as exp(scale s - LSE) ("flash-attention-v100"
// README: forward and backward passes for head dims up to 256, and a
// deterministic backward option). This is the deterministic form, with no
// atomics, in three kernels:
//   fa_bwd_pre_kernel   D per query row, and the LSE in log2 units (+inf for a
//                       row with no visible key and for the padding rows, so
//                       their P is exactly 0), stored [B][Hq][Nq rounded to 64];
//   fa_bwd_dkdv_kernel  one workgroup per 128 keys of a KV head, walking every
//                       query head of its group and every query tile; owns dK
//                       and dV of its keys. Orientation S = Q K^T: a lane owns a
//                       key, so P and dS leave the accumulators as the B
//                       operands of dV^T += dO^T P and dK^T += Q^T dS;
//   fa_bwd_dq_kernel    one workgroup per 128 query rows of a head, walking the
//                       key tiles; owns dQ of its rows. Orientation S^T = K Q^T
//                       as in the forward: dS^T feeds the B operand of
//                       dQ^T += K^T dS^T.
// The two passes recompute S and dP, seven tile products per (query, key) tile
// pair against five with a shared pass, and in exchange need no fp32 atomics
// and give bit-identical results from run to run.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D> struct BwdCfg {
  static constexpr int NW = 4;                      // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BT = 32;                     // rows of one tile (queries or keys)
  static constexpr int WROWS = NW * BT;             // rows a workgroup owns
  static constexpr int NS = D / 16;                 // 16-wide d slices
  static constexpr int NCB = D / 32;                // 32-wide d blocks
  // dK/dV workgroups per key block, each owning NCBO of the d blocks of dK and
  // dV (S and dP still contract over all of d): at d = 256 one wave's dK, dV,
  // K and V alone would take 384 of its 512 registers
  static constexpr int DSPLIT = D > 192 ? 2 : 1;
  static constexpr int NCBO = NCB / DSPLIT;
  static constexpr int TILE = BT * D * 2;           // bytes of one [32][D] tile
  static constexpr int BQ = 64;                     // query rows per step of the dK/dV pass
  static constexpr int TILEQ = BQ * D * 2;
  static constexpr int STW = 256;                   // floats of one wave's copy of a step's row statistics
  static_assert(STW * 4 == 64 * 16 && 2 * BQ <= STW, "one 16-byte DMA per lane fills a copy");
};

// DMA of [ROWS][D] row tiles (row pitch `pitch` bytes) into swizzled LDS. Piece
// i of this wave fills LDS bytes [(i NW + wave) 1024, +1024): lane l writes the
// 16 bytes at +16 l, physical chunk pch of row r, so it fetches logical chunk
// pch ^ swz(r) of that row. Bytes at or past `valid` read as zero.
template <int D, int ROWS> struct BwdDma {
  struct C {
    static constexpr int NW = BwdCfg<D>::NW;
    static constexpr int NPIECE = ROWS * D * 2 / 1024;   // 1 KB pieces per tile
    static constexpr int NDMA = (NPIECE + NW - 1) / NW;
    static constexpr bool EVEN = NPIECE % NW == 0;
    static_assert(ROWS * D * 2 % 1024 == 0, "tile must split into whole DMA pieces");
  };
  uint32_t goff[C::NDMA];
  int wave;
  __device__ __forceinline__ void init(uint32_t pitch, int wave_, int lane) {
    wave = wave_;
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i) {
      const uint32_t p = (i * C::NW + wave) * 1024 + lane * 16;
      const uint32_t r = p / (D * 2), pch = (p % (D * 2)) / 16;
      goff[i] = r * pitch + ((pch ^ Swz<D>::f(r)) << 4);
    }
  }
  __device__ __forceinline__ void issue(const char* base, int64_t valid, char* lds) const {
    const uint32_t nrec = valid > 0 ? static_cast<uint32_t>(valid > 0x7fffffff ? 0x7fffffff : valid) : 0u;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::NDMA; ++i)
      if (C::EVEN || i * C::NW + wave < C::NPIECE)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds + (i * C::NW + wave) * 1024), 16, goff[i], 0, 0, 0);
  }
};

// Two LDS stages of two row tiles each (Q and dO, or K and V), and for the
// dK/dV pass the row statistics of each stage (one copy per wave).
struct BwdLds {
  char* x[2];
  char* y[2];
  float* st[2];
};

// A-operand fragment of the rows of a swizzled [32][D] tile: 32 rows x d slice s.
template <int D, typename V8>
__device__ __forceinline__ V8 row_frag(const char* t, int s, int lane) {
  return lds_read_v8<V8>(t, Swz<D>::off(lane & 31, 2u * s + (lane >> 5)));
}

// Padded row count of the per-row statistics (whole dK/dV query tiles).
__host__ __device__ constexpr int bwd_nq_pad(int nq) { return (nq + 63) / 64 * 64; }

// The sequence of batch element b: its query and key counts and the first rows
// of its Q/dO/dQ and K/V/dK/dV in the (padded or packed) tensors, and the
// first entry of its LSE rows. A packed batch reads its bounds from the prefix
// sums, clamped into the tensors so that a malformed table cannot lead outside
// them. The row statistics are always [B][Hq][max rows rounded up to 64].
struct BwdSeq {
  int nq, nk;
  size_t q_row0, k_row0;
  __device__ __forceinline__ BwdSeq(const BwdArgs& a, int b) {
    if (a.cu_q != nullptr) {
      const int q_lo = min(max(a.cu_q[b], 0), a.total_q);
      const int q_hi = min(max(a.cu_q[b + 1], q_lo), a.total_q);
      const int k_lo = min(max(a.cu_k[b], 0), a.total_k);
      const int k_hi = min(max(a.cu_k[b + 1], k_lo), a.total_k);
      nq = min(q_hi - q_lo, a.Nq);
      nk = min(k_hi - k_lo, a.Nk);
      q_row0 = q_lo;
      k_row0 = k_lo;
    } else {
      nq = a.Nq;
      nk = a.Nk;
      q_row0 = static_cast<size_t>(b) * a.Nq;
      k_row0 = static_cast<size_t>(b) * a.Nk;
    }
  }
  // LSE of query head h, row i: [B][Hq][Nq], or [Hq][total_q] for a packed batch
  __device__ __forceinline__ size_t lse_index(const BwdArgs& a, int b, int h, int i) const {
    return a.cu_q != nullptr ? static_cast<size_t>(h) * a.total_q + q_row0 + i
                             : (static_cast<size_t>(b) * a.Hq + h) * a.Nq + i;
  }
};

// ---------------------------------------------------------------- preprocess

// G lanes per statistics entry (b, h, i), i < Nq rounded up to 64:
// D = sum_c dO * O in fp32 and the LSE in log2 units; padding rows and rows
// that saw no key get D = 0, LSE = +inf.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const BwdArgs a) {
  using T = typename Elem<BF16>::T;
  typedef T T8 __attribute__((ext_vector_type(8)));
  constexpr int CPR = D / 8;                              // 16-byte chunks per row
  constexpr int G = CPR <= 4 ? 4 : CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;
  constexpr int RPB = 256 / G;
  const int nqp = bwd_nq_pad(a.Nq);
  const int64_t entries = static_cast<int64_t>(a.B) * a.Hq * nqp;
  // thread groups enumerate (b, i, h) with the head fastest, so consecutive
  // groups read adjacent 16-byte chunks of the same [Hq][d] row of O and dO;
  // the statistics go to entry (b h) nqp + i
  const int64_t t = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / G;
  const int c = threadIdx.x % G;
  const int h = static_cast<int>(t % a.Hq);
  const int64_t bi = t / a.Hq;
  const int i = static_cast<int>(bi % nqp);
  const int b = static_cast<int>(bi / nqp);
  const int64_t e = (static_cast<int64_t>(b) * a.Hq + h) * nqp + i;
  const BwdSeq sq(a, t < entries ? b : 0);
  const bool live = t < entries && i < sq.nq;
  float acc = 0.f;
  if (live && c < CPR) {
    const int64_t row = ((static_cast<int64_t>(sq.q_row0) + i) * a.Hq + h) * D + 8 * c;
    const T8 o8 = *reinterpret_cast<const T8*>(reinterpret_cast<const T*>(a.o) + row);
    const T8 d8 = *reinterpret_cast<const T8*>(reinterpret_cast<const T*>(a.dout) + row);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc = __builtin_fmaf(static_cast<float>(o8[k]), static_cast<float>(d8[k]), acc);
  }
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, G);
  if (t < entries && c == 0) {
    float l2 = __builtin_huge_valf();
    if (live) {
      const float l = a.lse[sq.lse_index(a, b, h, i)];
      if (l != kNegInf) l2 = l * kLog2e;
    }
    a.dsum[e] = live ? acc : 0.f;
    a.lse2[e] = l2;
  }
}

// ---------------------------------------------------------------- dK, dV

template <int D, bool BF16, bool BAND> struct DkdvWave {
  using C = BwdCfg<D>;
  using E = Elem<BF16>;
  using T = typename E::T;
  using V8 = typename E::V8;

  const BwdArgs& a;
  const BwdSeq& sq;
  int lane, wave, hh;
  int b, g, key, k0w, diag;
  int cb0_;               // first d block of dK and dV this workgroup owns (see cb0)
  int nqt, t0, t1, nqp;   // query tiles [t0, t1) see some key of the workgroup
  int qlo, qspan;         // rows q that see this lane's key: 0 <= q - qlo <= qspan (unsigned)
  uint32_t qpitch;
  V8 kf[C::NS], vf[C::NS];          // this lane's key row of K and V (B operands)
  f32x16 dvt[C::NCBO], dkt[C::NCBO];  // dV^T and dK^T, [d][key], d blocks cb0 ..
  BwdDma<D, C::BQ> dma;

  __device__ __forceinline__ DkdvWave(const BwdArgs& args, const BwdSeq& seq, int b_, int g_, int k0, int dh)
      : a(args), sq(seq), b(b_), g(g_), cb0_(dh * C::NCBO) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    hh = lane >> 5;
    k0w = k0 + wave * C::BT;
    key = k0w + (lane & 31);
    diag = sq.nk - sq.nq;
    nqt = (sq.nq + C::BQ - 1) / C::BQ;
    nqp = bwd_nq_pad(a.Nq);
    // band: row q sees key j iff q + diag - wl <= j <= q + diag + wr (a side
    // at -1 is open; causal is (-1, 0)), so key j is seen by rows
    // j - diag - wr .. j - diag + wl
    const bool has_l = BAND && a.wl >= 0, has_r = BAND && a.wr >= 0;
    qlo = has_r ? key - diag - a.wr : -(1 << 29);
    qspan = (has_l ? key - diag + a.wl : (1 << 29)) - qlo;
    const int qa = has_r ? max(0, k0 - diag - a.wr) : 0;
    const int qb = has_l ? min(sq.nq - 1, k0 + C::WROWS - 1 - diag + a.wl) : sq.nq - 1;
    t0 = min(nqt, qa / C::BQ);
    t1 = qb >= qa ? min(nqt, qb / C::BQ + 1) : t0;
    qpitch = static_cast<uint32_t>(a.Hq) * D * 2;
    const size_t kv = ((sq.k_row0 + key) * a.Hkv + g) * D + 8 * hh;
    const T* kp = reinterpret_cast<const T*>(a.k) + kv;
    const T* vp = reinterpret_cast<const T*>(a.v) + kv;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      kf[s] = key < sq.nk ? *reinterpret_cast<const V8*>(kp + 16 * s) : V8{};
      vf[s] = key < sq.nk ? *reinterpret_cast<const V8*>(vp + 16 * s) : V8{};
    }
#pragma unroll
    for (int cb = 0; cb < C::NCBO; ++cb) {
      dvt[cb] = f32x16{};
      dkt[cb] = f32x16{};
    }
    dma.init(qpitch, wave, lane);
  }

  // Q and dO rows t*64 .. of query head hi of the group into one stage, and
  // their statistics into this wave's copy: the log2 LSE of the 64 rows, then
  // their D (lanes 0..15 and 16..31 move 16 bytes each, lanes 32..63 repeat
  // them). Branch-free, so that the DMA can sit among the MFMAs: when `live`
  // is false every range is empty, nothing is read and the stage is zeroed.
  __device__ __forceinline__ void fetch(int hi, int t, char* ql, char* ol, float* stl, bool live) const {
    const size_t off = ((sq.q_row0 + t * C::BQ) * a.Hq + g * a.group + hi) * D * 2;
    const int64_t valid = live ? static_cast<int64_t>(sq.nq - t * C::BQ - 1) * qpitch + D * 2 : 0;
    dma.issue(reinterpret_cast<const char*>(a.q) + off, valid, ql);
    dma.issue(reinterpret_cast<const char*>(a.dout) + off, valid, ol);
    {
      const uint32_t lse_off = static_cast<uint32_t>(reinterpret_cast<const char*>(a.lse2) -
                                                     reinterpret_cast<const char*>(a.dsum));
      const uint32_t row0 = ((b * a.Hq + g * a.group + hi) * nqp + t * C::BQ + 4 * (lane & 15)) * 4;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          a.dsum, 0, live ? lse_off + static_cast<uint32_t>(a.B * a.Hq * nqp) * 4 : 0u, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(stl + wave * C::STW), 16,
                                               ((lane & 31) < 16 ? lse_off : 0u) + row0, 0, 0, 0);
    }
  }

  // The 32 query rows from q0 of one half of a tile (tiles qt, ot in LDS, S and
  // dP already computed): P and dS with the query rows in registers (row
  // q0 + 8 (r / 4) + 4 hh + r % 4 in register r), then dV^T += dO^T P and
  // dK^T += Q^T dS over those rows. The transposed tiles come from v_frag, whose
  // row order matches the one the accumulator gives P and dS as B operands.
  template <bool MASK>
  __device__ __forceinline__ void half(int q0, const char* qt, const char* ot, const f32x4 (&l4)[4],
                                       const f32x4 (&d4)[4], const f32x16& s, const f32x16& dp) {
    f32x16 p, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(__builtin_fmaf(s[r], a.sl2, -l4[r >> 2][r & 3]));
      if (MASK) {
        const int q = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        pr = (static_cast<uint32_t>(q - qlo) > static_cast<uint32_t>(qspan)) ? 0.f : pr;
      }
      p[r] = pr;
      ds[r] = pr * (dp[r] - d4[r >> 2][r & 3]);
    }
    const V8 pf[2] = {to_v8<BF16>(p, 0), to_v8<BF16>(p, 8)};
    const V8 dsf[2] = {to_v8<BF16>(ds, 0), to_v8<BF16>(ds, 8)};
    // MFMA m: key slice u = m / (2 NCBO), d block cb0 + (m / 2) % NCBO, dV (even
    // m, dO^T fragment) or dK (odd m, Q^T fragment); fragments kTrPre MFMAs ahead
    V8 fr[kTrPre];
#pragma unroll
    for (int m = 0; m < kTrPre; ++m) fr[m] = tr_frag(qt, ot, m);
#pragma unroll
    for (int m = 0; m < kTrMf; ++m) {
      const int u = m / (2 * C::NCBO), cb = (m / 2) % C::NCBO;
      if (m & 1) dkt[cb] = E::mfma(fr[m % kTrPre], dsf[u], dkt[cb]);
      else dvt[cb] = E::mfma(fr[m % kTrPre], pf[u], dvt[cb]);
      if (m + kTrPre < kTrMf) fr[m % kTrPre] = tr_frag(qt, ot, m + kTrPre);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kTrPre, 0);
#pragma unroll
    for (int m = 0; m < kTrMf; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m + kTrPre < kTrMf) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
  // a compile-time 0 unless dK and dV are split over workgroups
  __device__ __forceinline__ int cb0() const { return C::DSPLIT > 1 ? cb0_ : 0; }
  static constexpr int kTrMf = 4 * C::NCBO;
  static constexpr int kTrPre = 3;
  __device__ __forceinline__ V8 tr_frag(const char* qt, const char* ot, int m) const {
    return v_frag<D, V8>((m & 1) ? qt : ot, cb0() + (m / 2) % C::NCBO, m / (2 * C::NCBO), lane);
  }

  // S = Q K^T and dP = dO V^T for both 32-row halves of a tile: MFMA m takes
  // the Q (even m) or dO (odd m) fragment of half m / (2 NS), d slice
  // (m / 2) % NS. Fragments are read kPre MFMAs ahead through a rolling buffer,
  // and the order is pinned for the scheduler, which otherwise issues each
  // read right before its MFMA when registers are tight.
  static constexpr int kSdMf = 4 * C::NS;
  static constexpr int kPre = 4;
  __device__ __forceinline__ V8 sd_frag(const char* qt, const char* ot, int m) const {
    return row_frag<D, V8>(((m & 1) ? ot : qt) + (m / (2 * C::NS)) * C::TILE, (m / 2) % C::NS, lane);
  }
  // The next tile's DMA (`hook`) goes out after MFMA kFetchAt, one instruction
  // per following MFMA. At d <= 64, whose two waves per SIMD leave no
  // registers for its addresses to stay live that long, the caller issues it
  // before the step's first MFMA instead (kFetchAt < 0: no hook call here).
  static constexpr int kFetchAt = D <= 64 ? -1 : 4;
  static constexpr int kFetchN = 2 * BwdDma<D, C::BQ>::C::NDMA + 1;   // DMA instructions of a fetch
  template <typename Hook>
  __device__ __forceinline__ void sdp(const char* qt, const char* ot, f32x16 (&s)[2], f32x16 (&dp)[2], Hook hook) const {
    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
    V8 fr[kPre];
#pragma unroll
    for (int m = 0; m < kPre; ++m) fr[m] = sd_frag(qt, ot, m);
#pragma unroll
    for (int m = 0; m < kSdMf; ++m) {
      const int h2 = m / (2 * C::NS), i = (m / 2) % C::NS;
      if (m & 1) dp[h2] = E::mfma(fr[m % kPre], vf[i], dp[h2]);
      else s[h2] = E::mfma(fr[m % kPre], kf[i], s[h2]);
      if (m + kPre < kSdMf) fr[m % kPre] = sd_frag(qt, ot, m + kPre);
      if (m == kFetchAt) hook();
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int m = 0; m < kSdMf; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m + kPre < kSdMf) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (kFetchAt >= 0 && m >= kFetchAt && m < kFetchAt + kFetchN) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
  }

  // Tile t (64 query rows) of query head hi, in stage ST: S = Q K^T and
  // dP = dO V^T for both 32-row halves first, so that the exponentials of one
  // half can overlap the products of the other. The next tile (in head-major
  // order; none after the last) is fetched into the other stage meanwhile.
  template <int ST, bool MASK>
  __device__ __forceinline__ void step(int hi, int t, const BwdLds& lds) {
    int hn = hi, tn = t + 1;
    if (tn == t1) {
      hn = hi + 1;
      tn = t0;
    }
    const bool live = hn < a.group;
    hn = live ? hn : 0;   // keeps the (unused) address inside the tensors
    if (kFetchAt < 0 && live) fetch(hn, tn, lds.x[ST ^ 1], lds.y[ST ^ 1], lds.st[ST ^ 1], true);
    const char* qt = lds.x[ST];
    const char* ot = lds.y[ST];
    // statistics of rows 32 h2 + 8 gq + 4 hh + 0..3, read before the pinned
    // phases so that only fragment reads are left for them to order (at d <= 64,
    // whose two waves per SIMD have no room for both halves' at once, each
    // half's right before its products)
    f32x4 l4[2][4], d4[2][4];
    auto stats = [&](int h2) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        l4[h2][gq] = *reinterpret_cast<const f32x4*>(lds.st[ST] + wave * C::STW + h2 * C::BT + 8 * gq + 4 * hh);
        d4[h2][gq] = *reinterpret_cast<const f32x4*>(lds.st[ST] + wave * C::STW + C::BQ + h2 * C::BT + 8 * gq + 4 * hh);
      }
    };
    if (D > 64) {
      stats(0);
      stats(1);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s[2], dp[2];
    sdp(qt, ot, s, dp, [&] { fetch(hn, tn, lds.x[ST ^ 1], lds.y[ST ^ 1], lds.st[ST ^ 1], live); });
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      if (D <= 64) stats(h2);
      half<MASK>(t * C::BQ + h2 * C::BT, qt + h2 * C::TILE, ot + h2 * C::TILE, l4[h2], d4[h2], s[h2], dp[h2]);
    }
    __syncthreads();
  }

  // tiles [t, te) of head hi; n counts the steps taken (stage = n & 1)
  template <bool MASK>
  __device__ __forceinline__ void run(int hi, int t, int te, int& n, const BwdLds& lds) {
    if (t < te && (n & 1)) {
      step<1, MASK>(hi, t, lds);
      ++t;
      ++n;
    }
    for (; t + 2 <= te; t += 2, n += 2) {
      step<0, MASK>(hi, t, lds);
      step<1, MASK>(hi, t + 1, lds);
    }
    if (t < te) {
      step<0, MASK>(hi, t, lds);
      ++n;
    }
  }

  // dV, and dK = scale (dK^T)^T, rounded to the element type (the workgroup's
  // d blocks of them). The wave's 32 key rows of each go through LDS (`stage`:
  // two swizzled [32][D] tiles of this wave alone), so that the global stores
  // write whole rows (half rows at d = 256), 16 bytes per lane with consecutive
  // lanes adjacent.
  __device__ __forceinline__ void finish(char* stage) const {
    typedef T T4 __attribute__((ext_vector_type(4)));
    const int ln32 = lane & 31;
#pragma unroll
    for (int cb = 0; cb < C::NCBO; ++cb)
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        T4 wv, wk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wv[e] = static_cast<T>(dvt[cb][4 * gr + e]);
          wk[e] = static_cast<T>(dkt[cb][4 * gr + e] * a.scale);
        }
        *reinterpret_cast<T4*>(stage + Swz<D>::off(ln32, 4 * (cb0() + cb) + gr) + 8 * hh) = wv;
        *reinterpret_cast<T4*>(stage + C::TILE + Swz<D>::off(ln32, 4 * (cb0() + cb) + gr) + 8 * hh) = wk;
      }
    wave_lds_sync();
    constexpr int CPR = 4 * C::NCBO;   // 16-byte chunks per row that this workgroup owns
    T* const dvb = reinterpret_cast<T*>(a.dv) + ((sq.k_row0 + k0w) * a.Hkv + g) * D;
    T* const dkb = reinterpret_cast<T*>(a.dk) + ((sq.k_row0 + k0w) * a.Hkv + g) * D;
#pragma unroll
    for (int i = 0; i < C::BT * CPR / 64; ++i) {
      const uint32_t c = 64 * i + lane;
      const uint32_t r = c / CPR, x = 4 * cb0() + c % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + Swz<D>::off(r, x));
      const u32x4 k = *reinterpret_cast<const u32x4*>(stage + C::TILE + Swz<D>::off(r, x));
      if (k0w + static_cast<int>(r) < sq.nk) {
        const size_t o = static_cast<size_t>(r) * a.Hkv * D + 8 * x;
        *reinterpret_cast<u32x4*>(dvb + o) = v;
        *reinterpret_cast<u32x4*>(dkb + o) = k;
      }
    }
  }
};

template <int D, bool BF16, bool BAND>
__global__ __launch_bounds__(BwdCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1, D <= 64 ? 2 : 1)))
void fa_bwd_dkdv_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char q_lds0[C::TILEQ];
  __shared__ __attribute__((aligned(1024))) char q_lds1[C::TILEQ];
  __shared__ __attribute__((aligned(1024))) char o_lds0[C::TILEQ];
  __shared__ __attribute__((aligned(1024))) char o_lds1[C::TILEQ];
  __shared__ __attribute__((aligned(16))) float st_lds0[C::NW * C::STW];
  __shared__ __attribute__((aligned(16))) float st_lds1[C::NW * C::STW];

  const int nkt = (a.Nk + C::WROWS - 1) / C::WROWS;
  int kt, gb;
  if (BAND) {
    // with a causal band the first key tiles see the most query rows
    blocked_order(blockIdx.x, nkt, a.Hkv * a.B, a.hb_kv, kt, gb);
  } else {
    xcd_heads(blockIdx.x, nkt, a.Hkv * a.B, gridDim.x, kt, gb);
  }
  const int g = gb % a.Hkv;
  const int b = gb / a.Hkv;
  const int k0 = kt * C::WROWS;
  const BwdSeq sq(a, b);
  if (k0 >= sq.nk) return;   // a packed sequence shorter than the grid: uniform, before any barrier
  DkdvWave<D, BF16, BAND> w(a, sq, b, g, k0, C::DSPLIT > 1 ? static_cast<int>(blockIdx.y) : 0);
  const BwdLds lds{{q_lds0, q_lds1}, {o_lds0, o_lds1}, {st_lds0, st_lds1}};

  // tiles [u0, u1) hold only rows that see every key of the workgroup; the
  // tiles before and after them (the band's edges) are computed with the mask
  int u0 = w.t0, u1 = w.t1;
  if (BAND) {
    const int ua = a.wr >= 0 ? k0 + C::WROWS - 1 - w.diag - a.wr : 0;   // first row seeing all keys
    const int ub = a.wl >= 0 ? k0 - w.diag + a.wl : (1 << 30);            // last such row
    u0 = min(w.t1, max(w.t0, ua > 0 ? (ua + C::BQ - 1) / C::BQ : 0));
    u1 = max(u0, min(w.t1, ub >= 0 ? (ub + 1) / C::BQ : 0));
  }
  w.fetch(0, w.t0, lds.x[0], lds.y[0], lds.st[0], w.t0 < w.t1);
  __syncthreads();
  int n = 0;
  for (int hi = 0; hi < a.group && w.t0 < w.t1; ++hi) {
    w.template run<true>(hi, w.t0, u0, n, lds);
    w.template run<false>(hi, u0, u1, n, lds);
    w.template run<true>(hi, u1, w.t1, n, lds);
  }
  __syncthreads();   // every wave is done with the last tile before the stages hold results
  {
    static_assert(C::NW == 4 && 2 * C::TILE <= C::TILEQ, "one stage buffer per wave holds its dV and dK rows");
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    w.finish(wv == 0 ? q_lds0 : wv == 1 ? q_lds1 : wv == 2 ? o_lds0 : o_lds1);
  }
}

// ---------------------------------------------------------------- dQ

template <int D, bool BF16, bool BAND> struct DqWave {
  using C = BwdCfg<D>;
  using E = Elem<BF16>;
  using T = typename E::T;
  using V8 = typename E::V8;

  const BwdArgs& a;
  const BwdSeq& sq;
  int lane, wave, hh;
  int b, hq, qrow, diag;
  int klo, kspan;            // keys k this lane's row sees: 0 <= k - klo <= kspan (unsigned), k < Nk
  int j0;                    // first key tile of the workgroup (its LDS stage 0)
  float lse2, dsum;
  const char* kg;
  const char* vg;
  int64_t valid;
  uint32_t kpitch;
  int nsteps;
  V8 qf[C::NS], of[C::NS];   // this lane's query row of Q and dO (B operands)
  f32x16 dqt[C::NCB];        // dQ^T, [d][q]
  BwdDma<D, C::BT> dma;

  __device__ __forceinline__ DqWave(const BwdArgs& args, const BwdSeq& seq, int b_, int hq_, int q0)
      : a(args), sq(seq), b(b_), hq(hq_) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    hh = lane >> 5;
    qrow = q0 + wave * C::BT + (lane & 31);
    diag = sq.nk - sq.nq;
    nsteps = 0;
    j0 = 0;
    const bool has_l = BAND && a.wl >= 0, has_r = BAND && a.wr >= 0;
    klo = has_l ? qrow + diag - a.wl : -(1 << 29);
    kspan = (has_r ? qrow + diag + a.wr : (1 << 29)) - klo;
    const bool live = qrow < sq.nq;
    const size_t r = ((sq.q_row0 + qrow) * a.Hq + hq) * D + 8 * hh;
    const T* qp = reinterpret_cast<const T*>(a.q) + r;
    const T* op = reinterpret_cast<const T*>(a.dout) + r;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      qf[s] = live ? *reinterpret_cast<const V8*>(qp + 16 * s) : V8{};
      of[s] = live ? *reinterpret_cast<const V8*>(op + 16 * s) : V8{};
    }
    const size_t si = (static_cast<size_t>(b) * a.Hq + hq) * bwd_nq_pad(a.Nq) + qrow;
    lse2 = live ? a.lse2[si] : __builtin_huge_valf();
    dsum = live ? a.dsum[si] : 0.f;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) dqt[cb] = f32x16{};
    kpitch = static_cast<uint32_t>(a.Hkv) * D * 2;
    const size_t head = (sq.k_row0 * a.Hkv + hq / a.group) * D * 2;
    kg = reinterpret_cast<const char*>(a.k) + head;
    vg = reinterpret_cast<const char*>(a.v) + head;
    valid = static_cast<int64_t>(sq.nk - 1) * kpitch + D * 2;
    dma.init(kpitch, wave, lane);
  }

  __device__ __forceinline__ void fetch(int j, char* kl, char* vl) const {
    const int64_t off = static_cast<int64_t>(j) * C::BT * kpitch;
    dma.issue(kg + off, valid - off, kl);
    dma.issue(vg + off, valid - off, vl);
  }

  // Key tile j (stage ST): S^T = K Q^T and dP^T = V dO^T with the keys in
  // registers (key 32 j + 8 (r / 4) + 4 hh + r % 4 in register r), then
  // dQ^T += K^T dS^T. The next key tile is fetched first. As in the dK/dV pass,
  // fragments are read a few MFMAs ahead and the order is pinned.
  static constexpr int kSdMf = 2 * C::NS;     // MFMA m: K (even) or V (odd) rows, d slice m / 2
  static constexpr int kPre = 4;
  static constexpr int kTrMf = 2 * C::NCB;    // MFMA m: key slice m / NCB, d block m % NCB
  static constexpr int kTrPre = 3;
  template <int ST, bool MASK>
  __device__ __forceinline__ void step(int j, const BwdLds& lds) {
    if (j + 1 < nsteps) fetch(j + 1, lds.x[ST ^ 1], lds.y[ST ^ 1]);
    const char* kt = lds.x[ST];
    const char* vt = lds.y[ST];
    f32x16 s = f32x16{}, dp = f32x16{};
    {
      V8 fr[kPre];
#pragma unroll
      for (int m = 0; m < kPre; ++m) fr[m] = row_frag<D, V8>((m & 1) ? vt : kt, m / 2, lane);
#pragma unroll
      for (int m = 0; m < kSdMf; ++m) {
        if (m & 1) dp = E::mfma(fr[m % kPre], of[m / 2], dp);
        else s = E::mfma(fr[m % kPre], qf[m / 2], s);
        if (m + kPre < kSdMf) fr[m % kPre] = row_frag<D, V8>(((m + kPre) & 1) ? vt : kt, (m + kPre) / 2, lane);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
      for (int m = 0; m < kSdMf; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m + kPre < kSdMf) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(__builtin_fmaf(s[r], a.sl2, -lse2));
      if (MASK) {
        const int kk = j * C::BT + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool hide = kk >= sq.nk || (BAND && static_cast<uint32_t>(kk - klo) > static_cast<uint32_t>(kspan));
        pr = hide ? 0.f : pr;
      }
      ds[r] = pr * (dp[r] - dsum);
    }
    const V8 dsf[2] = {to_v8<BF16>(ds, 0), to_v8<BF16>(ds, 8)};
    {
      V8 fr[kTrPre];
#pragma unroll
      for (int m = 0; m < kTrPre; ++m) fr[m] = v_frag<D, V8>(kt, m % C::NCB, m / C::NCB, lane);
#pragma unroll
      for (int m = 0; m < kTrMf; ++m) {
        dqt[m % C::NCB] = E::mfma(fr[m % kTrPre], dsf[m / C::NCB], dqt[m % C::NCB]);
        if (m + kTrPre < kTrMf) fr[m % kTrPre] = v_frag<D, V8>(kt, (m + kTrPre) % C::NCB, (m + kTrPre) / C::NCB, lane);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kTrPre, 0);
#pragma unroll
      for (int m = 0; m < kTrMf; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m + kTrPre < kTrMf) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    __syncthreads();
  }

  // key tiles [j, je), tile j in stage (j - j0) & 1
  template <bool MASK>
  __device__ __forceinline__ void run(int j, int je, const BwdLds& lds) {
    if (j < je && ((j - j0) & 1)) {
      step<1, MASK>(j, lds);
      ++j;
    }
    for (; j + 2 <= je; j += 2) {
      step<0, MASK>(j, lds);
      step<1, MASK>(j + 1, lds);
    }
    if (j < je) step<0, MASK>(j, lds);
  }

  __device__ __forceinline__ void finish() const {
    if (qrow >= sq.nq) return;
    T* dqp = reinterpret_cast<T*>(a.dq) + ((sq.q_row0 + qrow) * a.Hq + hq) * D;
    typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = static_cast<T>(dqt[cb][4 * gr + e] * a.scale);
        *reinterpret_cast<T4*>(dqp + 32 * cb + 8 * gr + 4 * hh) = w;
      }
  }
};

template <int D, bool BF16, bool BAND>
__global__ __launch_bounds__(BwdCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : D <= 128 ? 2 : 1, D <= 64 ? 3 : D <= 128 ? 2 : 1)))
void fa_bwd_dq_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k_lds1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds1[C::TILE];

  const int nqt = (a.Nq + C::WROWS - 1) / C::WROWS;
  int qt, hb;
  if (BAND) {
    // with a causal band the last query tiles see the most keys
    int o;
    blocked_order(blockIdx.x, nqt, a.Hq * a.B, a.hb_q, o, hb, a.group);
    qt = nqt - 1 - o;
  } else {
    xcd_heads(blockIdx.x, nqt, a.Hq * a.B, gridDim.x, qt, hb, a.group);
  }
  const int hq = hb % a.Hq;
  const int b = hb / a.Hq;
  const int q0 = qt * C::WROWS;
  const BwdSeq sq(a, b);
  if (q0 >= sq.nq) return;   // a packed sequence shorter than the grid: uniform, before any barrier
  DqWave<D, BF16, BAND> w(a, sq, b, hq, q0);
  const BwdLds lds{{k_lds0, k_lds1}, {v_lds0, v_lds1}, {nullptr, nullptr}};

  // key tiles [j0, nsteps) hold a key some row of the workgroup sees; tiles
  // [u0, u1) hold only keys every row sees (below Nk); the others are masked
  const int last = min(q0 + C::WROWS, sq.nq) - 1;
  const bool has_l = BAND && a.wl >= 0, has_r = BAND && a.wr >= 0;
  const int ka = has_l ? max(0, q0 + w.diag - a.wl) : 0;
  const int kb = has_r ? min(sq.nk - 1, last + w.diag + a.wr) : sq.nk - 1;
  w.j0 = ka / C::BT;
  w.nsteps = kb >= ka ? kb / C::BT + 1 : w.j0;
  const int ua = has_l ? max(0, last + w.diag - a.wl) : 0;
  const int ub = min(sq.nk - 1, has_r ? q0 + w.diag + a.wr : sq.nk - 1);
  const int u0 = min(w.nsteps, max(w.j0, (ua + C::BT - 1) / C::BT));
  const int u1 = max(u0, min(w.nsteps, ub >= 0 ? (ub + 1) / C::BT : 0));

  if (w.nsteps > w.j0) w.fetch(w.j0, lds.x[0], lds.y[0]);
  __syncthreads();
  w.template run<true>(w.j0, u0, lds);
  w.template run<false>(u0, u1, lds);
  w.template run<true>(u1, w.nsteps, lds);
  w.finish();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool bf16, bool band, hipStream_t stream) {
  using C = BwdCfg<D>;
  (void)hipGetLastError();   // start from a clean error state
  {
    constexpr int CPR = D / 8;
    constexpr int G = CPR <= 4 ? 4 : CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;
    const int64_t entries = static_cast<int64_t>(a.B) * a.Hq * bwd_nq_pad(a.Nq);
    const dim3 grid(static_cast<unsigned>((entries + 256 / G - 1) / (256 / G)));
    if (bf16) fa_bwd_pre_kernel<D, true><<<grid, 256, 0, stream>>>(a);
    else fa_bwd_pre_kernel<D, false><<<grid, 256, 0, stream>>>(a);
  }
  const dim3 block(C::THREADS);
  const dim3 grid_kv(static_cast<unsigned>((a.Nk + C::WROWS - 1) / C::WROWS) * a.Hkv * a.B, C::DSPLIT);
  const dim3 grid_q(static_cast<unsigned>((a.Nq + C::WROWS - 1) / C::WROWS) * a.Hq * a.B);
  if (bf16) {
    if (band) {
      fa_bwd_dkdv_kernel<D, true, true><<<grid_kv, block, 0, stream>>>(a);
      fa_bwd_dq_kernel<D, true, true><<<grid_q, block, 0, stream>>>(a);
    } else {
      fa_bwd_dkdv_kernel<D, true, false><<<grid_kv, block, 0, stream>>>(a);
      fa_bwd_dq_kernel<D, true, false><<<grid_q, block, 0, stream>>>(a);
    }
  } else {
    if (band) {
      fa_bwd_dkdv_kernel<D, false, true><<<grid_kv, block, 0, stream>>>(a);
      fa_bwd_dq_kernel<D, false, true><<<grid_q, block, 0, stream>>>(a);
    } else {
      fa_bwd_dkdv_kernel<D, false, false><<<grid_kv, block, 0, stream>>>(a);
      fa_bwd_dq_kernel<D, false, false><<<grid_q, block, 0, stream>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace fa
