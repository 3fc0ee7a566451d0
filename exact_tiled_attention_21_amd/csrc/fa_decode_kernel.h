// Split-KV attention for decode (Flash-Decoding) on gfx950.
//
// "flash-attention-v100" README, Changelog 2.2: with very short query blocks
// the cost is reading the KV cache, so the key range is split over several
// workgroups and a separate kernel merges the results. The "flash attention-2
// github" search page spells out the steps: split K/V into chunks, attend to
// every chunk in parallel while writing one extra scalar per row and chunk
// (the log-sum-exp), then combine.
//
// Split kernel: the keys are cut into 32-key tiles and dealt out to the parts
// round-robin: part p of P*S parts takes tiles p, p + P*S, ... (S requested
// splits, each dealt out as P = 1, 2 or 4 parts so that the chip gets about one
// round of waves). Any partition of the keys merges exactly, and this one makes
// the parts of a sequence read one dense window of the cache at a time (all
// parts step through neighbouring tiles together), which keeps the DRAM pages
// open: with contiguous chunks every part streams its own region. One
// single-wave workgroup per (part, KV head, batch[, row block]) (two waves at
// d = 256, splitting the tile's loads and O's columns); the query rows
// of the whole GQA group (Hq/Hkv heads x Nq positions, at most 32 per row block)
// share the part's K/V, which is therefore read from HBM once. The wave loads
// each tile with fully coalesced, non-temporal 16-byte loads into registers
// (one tile ahead, except at d = 192: about 16 MiB in flight chip-wide is
// enough for the HBM rate, more only thins out the DRAM locality), stages it
// through its own swizzled LDS tiles (K for the A operand, V for the
// transposing read), and writes one normalised fp32 partial and its
// log-sum-exp per row; the combine kernel merges the partials. No barriers
// between single waves: up to four share a CU, one per SIMD.
//
// Paged cache ("flash-attention-v100" README, flash_attn_with_kvcache: a block
// table maps each sequence's logical key blocks to pages of a shared pool, and
// cache_seqlens gives each sequence's length): a 32-key tile never straddles a
// page (the page size is a multiple of 32), so each tile costs one block-table
// read and otherwise loads exactly like a contiguous tile. The tiles dealt out
// are those below each sequence's own length, and the causal mask is aligned
// to it.
//
// Combine kernel: per output row, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s; parts with LSE_s = -inf weigh nothing.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D> struct DecCfg {
  static constexpr int BC = 32;                   // keys per tile
  static constexpr int NS = D / 16;               // 16-wide d slices (QK^T depth)
  static constexpr int NCB = D / 32;              // 32-wide d blocks of O^T
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int NCH = BC * CPR / 64;       // 16-byte chunks per lane per tensor per tile
  // waves per workgroup: at d = 256 two waves share the tile (each loads half of
  // it) and each accumulates half of O's d blocks; both compute all the scores
  static constexpr int NWV = D > 192 ? 2 : 1;
  static constexpr int NCBO = NCB / NWV;          // d blocks of O^T per wave
  static constexpr int NCHW = NCH / NWV;          // chunks per lane per tensor per tile per wave
  // the next tile's loads go out before the current tile's products when a
  // wave's share of a tile is at most 8 chunks per tensor; more (d = 192), live
  // across those products, would spill
  static constexpr bool AHEAD = NCHW <= 8;
  static_assert(NCB % NWV == 0 && NCH % NWV == 0, "the waves split O and the tile evenly");
  static constexpr int TILE = BC * D * 2;         // bytes of one K or V tile
};

// Cache policy of the K/V loads: non-temporal (every cache byte is read exactly
// once per step, so it should not displace anything).
constexpr int kNonTemporal = 2;

// One wave per workgroup: it streams the tiles of one part.
template <int D, bool BF16, bool CAUSAL, bool PAGED> struct DecWave {
  using C = DecCfg<D>;
  using E = Elem<BF16>;
  using T = typename E::T;
  using V8 = typename E::V8;
  typedef u32x4 Stage[C::NCHW];

  const DecodeArgs& a;
  int lane, hh, wv;             // wv: this wave's index in the workgroup
  bool rvalid;
  int b, g, L;                  // batch, KV head, keys of this sequence
  int ri, rhq, diag, i_first, k_hi, ntile;
  int part, nparts;             // this part's index and the number of parts (tile stride)
  float sl2;
  V8 qf[C::NS];
  f32x16 oacc[C::NCBO];         // O^T, d blocks wv NCBO ..
  float m_run, l_part;
  const char* kg;
  const char* vg;
  uint32_t rowbytes;
  int64_t valid;
  uint32_t goff;                // this lane's first 16-byte piece of a tile (coalesced rows)
  uint32_t kro, kxo, vb0, vb1, vx0, vx1;   // LDS fragment read offsets

  __device__ __forceinline__ DecWave(const DecodeArgs& args, int part_, int g_, int rb, int b_)
      : a(args), b(b_), g(g_) {
    lane = threadIdx.x & 63;
    hh = lane >> 5;
    wv = C::NWV > 1 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) : 0;
    const int R = a.group * a.Nq;               // rows of this KV head group
    L = a.Nk;
    if (PAGED) L = min(max(a.seqlens[b], 0), a.max_pages * a.page_size);
    diag = L - a.Nq;
    // row r = i * group + (hq - g * group): consecutive rows are adjacent heads
    const int r = rb * 32 + (lane & 31);
    rvalid = r < R;
    ri = rvalid ? r / a.group : 0;
    rhq = g * a.group + (rvalid ? r % a.group : 0);
    sl2 = a.sl2;
    const T* qp = reinterpret_cast<const T*>(a.q) +
                  ((static_cast<size_t>(b) * a.Nq + ri) * a.Hq + rhq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) qf[s] = rvalid ? *reinterpret_cast<const V8*>(qp + 16 * s) : V8{};
    // a negative scale: scores of -q against |scale|, so the row max taken below is
    // the max of the scaled scores
    if (a.negate_q) {
#pragma unroll
      for (int s = 0; s < C::NS; ++s) qf[s] = -qf[s];
    }

    // tiles of this part: the keys are cut into 32-key tiles and part p of the
    // nparts parts takes tiles p, p + nparts, p + 2 nparts, ... below k_hi (the
    // sequence length, or for causal one past the last row's last key)
    part = part_;
    nparts = a.splits;
    i_first = (rb * 32) / a.group;
    k_hi = L;
    if (CAUSAL) {
      const int i_last = (min(R, rb * 32 + 32) - 1) / a.group;
      k_hi = max(0, min(k_hi, i_last + diag + 1));
    }
    const int tiles = (k_hi + C::BC - 1) / C::BC;
    ntile = part < tiles ? (tiles - part + nparts - 1) / nparts : 0;

    rowbytes = static_cast<uint32_t>(a.Hkv) * D * 2;
    const size_t head_off = ((PAGED ? 0 : static_cast<size_t>(b) * a.Nk * a.Hkv) + g) * D * 2;
    kg = reinterpret_cast<const char*>(a.k) + head_off;
    vg = reinterpret_cast<const char*>(a.v) + head_off;
    valid = static_cast<int64_t>(a.Nk - 1) * rowbytes + D * 2;
    // offset of this lane's first piece of a tile (see goff_of)
    goff = static_cast<uint32_t>(lane / C::CPR) * rowbytes + static_cast<uint32_t>(lane % C::CPR) * 16;

    kro = static_cast<uint32_t>(lane & 31) * (D * 2);
    kxo = (static_cast<uint32_t>(hh) ^ Swz<D>::f(lane & 31)) << 4;
    const uint32_t vj = lane & 15, vcb = (lane >> 4) & 1;
    const uint32_t vrow0 = 4 * hh + (vj >> 2), vrow1 = vrow0 + 8;
    const uint32_t vxl = 2 * vcb + ((vj & 3) >> 1);
    vx0 = (vxl ^ Swz<D>::f(vrow0)) << 4;
    vx1 = (vxl ^ Swz<D>::f(vrow1)) << 4;
    vb0 = vrow0 * (D * 2) + 8 * (vj & 1);
    vb1 = vrow1 * (D * 2) + 8 * (vj & 1);
#pragma unroll
    for (int cb = 0; cb < C::NCBO; ++cb) oacc[cb] = f32x16{};
    m_run = kNegInf;
    l_part = 0.f;
  }

  // first key of this part's tile t
  __device__ __forceinline__ int key0_of(int t) const { return (part + t * nparts) * C::BC; }

  // K and V rows of tile t into registers, 16 lanes per 256-byte row (coalesced);
  // rows past the sequence read as zero through the buffer bounds check. A
  // paged tile lies in one page; a page index outside the pool reads as zeros
  // rather than leaving the pool.
  __device__ __forceinline__ void load(int t, Stage& ks, Stage& vs) const {
    const int key0 = key0_of(t);
    int64_t off, rem;
    if (PAGED) {
      const int rows = min(C::BC, L - key0);
      int page = -1;
      if (rows > 0) page = a.block_table[static_cast<size_t>(b) * a.max_pages + key0 / a.page_size];
      const bool ok = rows > 0 && page >= 0 && page < a.num_pages;
      off = ok ? (static_cast<int64_t>(page) * a.page_size + key0 % a.page_size) * rowbytes : 0;
      rem = ok ? static_cast<int64_t>(rows - 1) * rowbytes + D * 2 : 0;
    } else {
      off = static_cast<int64_t>(key0) * rowbytes;
      rem = valid - off;
      if (rem <= 0) off = 0;
    }
    const uint32_t nrec = rem > 0 ? static_cast<uint32_t>(rem > 0x7fffffff ? 0x7fffffff : rem) : 0u;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kg + off), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vg + off), 0, nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < C::NCHW; ++j) {
      const uint32_t o = goff_of(wv * C::NCHW + j);
      ks[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, kNonTemporal));
      vs[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, kNonTemporal));
    }
  }
  // piece i of a tile is 16-byte chunk c = lane + 64 i of the tile: row c / CPR, chunk c % CPR
  static constexpr bool kEvenRows = (64 % C::CPR) == 0;   // d = 32, 64, 128, 256
  __device__ __forceinline__ uint32_t goff_of(int i) const {
    if (kEvenRows) return goff + static_cast<uint32_t>((64 * i) / C::CPR) * rowbytes;
    const uint32_t c = lane + 64 * i;
    return (c / C::CPR) * rowbytes + (c % C::CPR) * 16;
  }
  // registers -> the workgroup's swizzled LDS tiles (this wave's pieces)
  __device__ __forceinline__ void stage(const Stage& ks, const Stage& vs, char* kt, char* vt) const {
#pragma unroll
    for (int j = 0; j < C::NCHW; ++j) {
      const int i = wv * C::NCHW + j;
      const uint32_t c = lane + 64 * i;
      const uint32_t o = Swz<D>::off(c / C::CPR, c % C::CPR);
      *reinterpret_cast<u32x4*>(kt + o) = ks[j];
      *reinterpret_cast<u32x4*>(vt + o) = vs[j];
    }
  }
  __device__ __forceinline__ V8 kfrag(const char* kt, int s) const {
    return lds_read_v8<V8>(kt, (kxo ^ (32u * s)) + kro);
  }
  __device__ __forceinline__ V8 vfrag(const char* vt, int cb, int t) const {
    const uint32_t lo = t * 16 * (D * 2) + ((vx0 ^ (64u * cb)) + vb0);
    const uint32_t hi = t * 16 * (D * 2) + ((vx1 ^ (64u * cb)) + vb1);
    return __builtin_bit_cast(V8, __builtin_shufflevector(lds_read_tr(vt, lo), lds_read_tr(vt, hi),
                                                          0, 1, 2, 3, 4, 5, 6, 7));
  }

  // one 32-key tile from the LDS tiles: scores, online softmax, O += V P
  template <bool MASK>
  __device__ __forceinline__ void tile(int t, const char* kt, const char* vt) {
    const int k0 = key0_of(t);
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < C::NS; ++s) sacc = E::mfma(kfrag(kt, s), qf[s], sacc);
    if (MASK) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int key = k0 + 8 * (q >> 2) + 4 * hh + (q & 3);
        if (key >= k_hi || (CAUSAL && key > ri + diag)) sacc[q] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, sacc[q]);
    mx = halves_max(mx);
    const float mxs = (mx == kNegInf) ? kNegInf : mx * sl2;
    const bool need = mxs > m_run + 8.0f;   // reference max moves by more than 2^8 (or is set)
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      const float m_new = need ? mxs : m_run;
      const float alpha = (m_new == m_run) ? 1.f : exp2_fast(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int cb = 0; cb < C::NCBO; ++cb) oacc[cb] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float psum[2] = {0.f, 0.f};
    f32x16 p;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float e = exp2_fast(__builtin_fmaf(sacc[q], sl2, -m_use));
      if (MASK) e = (sacc[q] == kNegInf) ? 0.f : e;
      p[q] = e;
      psum[q & 1] += e;
    }
    l_part += psum[0] + psum[1];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const V8 pf = to_v8<BF16>(p, 8 * tt);
#pragma unroll
      for (int cb = 0; cb < C::NCBO; ++cb) oacc[cb] = E::mfma(vfrag(vt, wv * C::NCBO + cb, tt), pf, oacc[cb]);
    }
  }
  __device__ __forceinline__ void tile_any(int t, const char* kt, const char* vt) {
    const int k0 = key0_of(t);
    if ((k0 + C::BC > k_hi) || (CAUSAL && k0 + C::BC - 1 > i_first + diag)) tile<true>(t, kt, vt);
    else tile<false>(t, kt, vt);
  }
};

// LDS hand-over between the workgroup's waves: the wave's own when it is alone
template <int NWV>
__device__ __forceinline__ void dec_lds_sync() {
  if (NWV > 1) __syncthreads();
  else wave_lds_sync();
}

template <int D, bool BF16, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(64 * DecCfg<D>::NWV) void fa_decode_split_kernel(const DecodeArgs a) {
  using C = DecCfg<D>;
  using W = DecWave<D, BF16, CAUSAL, PAGED>;
  __shared__ __attribute__((aligned(1024))) char kt[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vt[C::TILE];

  // the batch index is the grid's fastest axis, so the workgroups of one
  // sequence share an XCD (workgroup ids go to the XCDs round-robin): the KV
  // heads of a cache row, which interleave in memory, are then all read from
  // one XCD (with a single sequence, the heads of one part are)
  const int part = blockIdx.y;            // one of the a.splits parts
  const int g = blockIdx.z % a.Hkv;
  const int rb = blockIdx.z / a.Hkv;
  const int b = blockIdx.x;
  W w(a, part, g, rb, b);

  // tiles t of this part: the loads of tile t + 1 are issued once tile t sits in
  // LDS, so they overlap tile t's products (d = 192 loads each tile right before
  // staging it and relies on the other waves of the CU);
  // loads past the end read zeros, so each tile's wait covers exactly its own loads
  typename W::Stage ks, vs;
  if (C::AHEAD) w.load(0, ks, vs);
  for (int t = 0; t < w.ntile; ++t) {
    if (!C::AHEAD) w.load(t, ks, vs);
    w.stage(ks, vs, kt, vt);
    dec_lds_sync<C::NWV>();
    if (C::AHEAD) w.load(t + 1, ks, vs);
    w.tile_any(t, kt, vt);
    dec_lds_sync<C::NWV>();
  }

  // normalised partial and its log2-sum-exp; a part with no visible key
  // writes O = 0, LSE = -inf
  const float l = halves_sum(w.l_part);
  if (!w.rvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t prow = ((static_cast<size_t>(part) * a.B + b) * a.Hq + w.rhq) * a.Nq + w.ri;
  float* po = a.part_o + prow * D;
#pragma unroll
  for (int cb = 0; cb < C::NCBO; ++cb)
#pragma unroll
    for (int gr = 0; gr < 4; ++gr) {
      f32x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = w.oacc[cb][4 * gr + e] * inv;
      *reinterpret_cast<f32x4*>(po + 32 * (w.wv * C::NCBO + cb) + 8 * gr + 4 * w.hh) = o4;
    }
  if (w.hh == 0 && w.wv == 0) a.part_lse[prow] = l > 0.f ? w.m_run + __log2f(l) : kNegInf;
}

// One row of the output per D/4 threads: O = sum_s w_s O_s with
// w_s = exp(LSE_s - LSE), LSE = log sum_s exp(LSE_s) (log2 domain inside).
// One pass: the LSEs and partial outputs of 16 parts are loaded together and
// merged against a running max, so a step with at most 16 parts waits on memory
// once.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(const DecodeArgs a) {
  using T = typename Elem<BF16>::T;
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  constexpr int SB = 16;
  const int rows = a.B * a.Hq * a.Nq;
  // the batch varies fastest over the workgroups, like in the split kernel, so
  // batch b's partials are merged on the XCD that wrote them
  const int rows_b = a.Hq * a.Nq;
  const int rloc = (blockIdx.x / a.B) * RPB + threadIdx.x / TPR;
  if (rloc >= rows_b) return;
  const int row = (blockIdx.x % a.B) * rows_b + rloc;
  const int c4 = (threadIdx.x % TPR) * 4;
  const size_t stride = static_cast<size_t>(rows);   // elements between parts
  float mx = kNegInf;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += SB) {
    float l[SB];
    f32x4 o[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const bool ok = s0 + i < a.splits;
      l[i] = ok ? a.part_lse[(s0 + i) * stride + row] : kNegInf;
      o[i] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + ((s0 + i) * stride + row) * D + c4)
                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = kNegInf;
#pragma unroll
    for (int i = 0; i < SB; ++i) mb = fmaxf(mb, l[i]);
    if (mb == kNegInf) continue;   // no part of this batch saw a key
    if (mb > mx) {                 // move the reference: earlier weights shrink (to 0 from -inf)
      const float r = exp2_fast(mx - mb);
      acc *= r;
      tot *= r;
      mx = mb;
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const float wgt = exp2_fast(l[i] - mx);   // 0 for a part with no key (-inf)
      tot += wgt;
      acc += wgt * o[i];
    }
  }
  if (mx != kNegInf) acc *= 1.f / tot;
  // row = (b * Hq + hq) * Nq + i  ->  o[b][i][hq][:]
  const int i = row % a.Nq;
  const int bh = row / a.Nq;
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (T)acc[e];
  *reinterpret_cast<T4*>(reinterpret_cast<T*>(a.o) + ((static_cast<size_t>(b) * a.Nq + i) * a.Hq + hq) * D + c4) = w;
  if (a.lse != nullptr && c4 == 0) a.lse[row] = (mx == kNegInf) ? kNegInf : (mx + __log2f(tot)) * kLn2;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bool bf16, bool causal, hipStream_t stream) {
  using C = DecCfg<D>;
  const dim3 grid1(a.B, a.splits, a.Hkv * a.row_blocks);   // a.splits = all parts
  (void)hipGetLastError();   // start from a clean error state
  const bool paged = a.block_table != nullptr;
#define FA_DEC_SPLIT(BF, CA)                                                     \
  do {                                                                           \
    if (paged) fa_decode_split_kernel<D, BF, CA, true><<<grid1, 64 * C::NWV, 0, stream>>>(a); \
    else fa_decode_split_kernel<D, BF, CA, false><<<grid1, 64 * C::NWV, 0, stream>>>(a);      \
  } while (0)
  if (bf16) {
    if (causal) FA_DEC_SPLIT(true, true);
    else FA_DEC_SPLIT(true, false);
  } else {
    if (causal) FA_DEC_SPLIT(false, true);
    else FA_DEC_SPLIT(false, false);
  }
#undef FA_DEC_SPLIT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (D / 4);
  const dim3 grid2(static_cast<unsigned>(a.B) * ((a.Hq * a.Nq + RPB - 1) / RPB));
  if (bf16) fa_decode_combine_kernel<D, true><<<grid2, 256, 0, stream>>>(a);
  else fa_decode_combine_kernel<D, false><<<grid2, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fa
