// Device building blocks for exact tiled attention on gfx950 (CDNA4, wave64).
//
// The score tile is computed transposed, S^T = K Q^T, on the 32x32x16 MFMA:
// the accumulator gives every lane one query column (lane & 31) and 16 of the
// tile's keys, so a row's max and sum are in-lane reductions plus one exchange
// between the two 32-lane halves (v_permlane32_swap). The probabilities P stay
// in those registers and feed the B operand of O^T += V^T P^T directly; the
// V^T operand is fetched from a row-major [key][d] LDS tile with the gfx950
// transposing read ds_read_b64_tr_b16, so V is never transposed in memory.
//
// Operand layouts of v_mfma_f32_32x32x16_{f16,bf16} (lane l, half h = l >> 5):
//   A (32 x 16): lane l holds A[l & 31][8h .. 8h+7]
//   B (16 x 32): lane l holds B[8h .. 8h+7][l & 31]
//   C (32 x 32): lane l, register r holds C[8(r/4) + 4h + (r%4)][l & 31]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Element type traits: the 8-wide MFMA operand and the MFMA itself.
template <bool BF16> struct Elem;
template <> struct Elem<false> {
  typedef _Float16 T;
  typedef f16x8 V8;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Elem<true> {
  typedef __bf16 T;
  typedef bf16x8 V8;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// XOR swizzle of the 16-byte chunks of a row-major [rows][D] b16 LDS tile.
// Physical chunk = logical chunk ^ swz(row), with row bit 0 -> bit 3,
// bit 1 -> bit 2, bits 2..3 -> bits 0..1, masked to stay inside the aligned
// power-of-two group of chunks that every row owns (4 chunks for d = 32 and
// 96, 8 for 64 and 192, 16 for 128 and 256). Against 64 banks of 4 bytes this
// makes both the A-operand reads of K (16 lanes reading one chunk of 16
// consecutive rows) and the transposing reads of V (32 lanes reading 64 bytes
// of 4 consecutive rows) conflict-free.
template <int D> struct Swz {
  static constexpr uint32_t kChunks = D / 8;
  static constexpr uint32_t kMask = (kChunks % 16 == 0) ? 15u : (kChunks % 8 == 0) ? 7u : 3u;
  static __device__ __forceinline__ uint32_t f(uint32_t row) {
    return (((row & 1u) << 3) | ((row & 2u) << 1) | ((row >> 2) & 3u)) & kMask;
  }
  // byte offset of (row, logical 16-byte chunk x) inside a tile
  static __device__ __forceinline__ uint32_t off(uint32_t row, uint32_t x) {
    return row * (uint32_t)(D * 2) + ((x ^ f(row)) << 4);
  }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x in the other 32-lane half (same query column): max/sum helpers.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename V8>
__device__ __forceinline__ V8 lds_read_v8(const char* lds, uint32_t off) {
  return *reinterpret_cast<const V8*>(lds + off);
}

// Transposing LDS read: within each 16-lane group, 4 rows x 16 columns of b16
// come back as 16 lanes x 4 rows (lane j gets column j of the 4 rows).
__device__ __forceinline__ i16x4 lds_read_tr(const char* lds, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + off));
}

// A-operand fragment of V^T for the P V product: c-block cb (32 head-dim
// columns) and key slice t (16 keys). Lane (c = 32cb + (l & 31), half h)
// receives keys 16t + 4h + 0..3 and 16t + 8 + 4h + 0..3 at column c, which is
// exactly the key order the S^T accumulator gives P in its B operand.
template <int D, typename V8>
__device__ __forceinline__ V8 v_frag(const char* vt, int cb, int t, int lane) {
  const uint32_t j = lane & 15, cblk = (lane >> 4) & 1, h = lane >> 5;
  const uint32_t x = 4u * cb + 2u * cblk + ((j & 3u) >> 1);
  const uint32_t r0 = 16u * t + 4u * h + (j >> 2);
  const uint32_t lo = Swz<D>::off(r0, x) + 8u * (j & 1u);
  const uint32_t hi = Swz<D>::off(r0 + 8u, x) + 8u * (j & 1u);
  i16x4 a = lds_read_tr(vt, lo);
  i16x4 b = lds_read_tr(vt, hi);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(V8, w);
}

// A-operand fragment of K for S^T = K Q^T: key block kb (32 keys), d-slice s.
template <int D, typename V8>
__device__ __forceinline__ V8 k_frag(const char* kt, int kb, int s, int lane) {
  const uint32_t row = 32u * kb + (lane & 31);
  return lds_read_v8<V8>(kt, Swz<D>::off(row, 2u * s + (lane >> 5)));
}

// Rounds 8 fp32 values to the element type (nearest even) as an MFMA operand.
template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::V8 to_v8(const f32x16& x, int base) {
  typename Elem<BF16>::V8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (typename Elem<BF16>::T)x[base + i];
  return r;
}

// acc + x[2i] + x[2i+1] on the packed pair i of an 8-wide operand (fp32 sum)
template <bool BF16>
__device__ __forceinline__ float dot2_ones(typename Elem<BF16>::V8 x, int i, float acc);
template <>
__device__ __forceinline__ float dot2_ones<false>(f16x8 x, int i, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
  const h2 v = {x[2 * i], x[2 * i + 1]};
  return __builtin_amdgcn_fdot2(v, one, acc, false);
}
template <>
__device__ __forceinline__ float dot2_ones<true>(bf16x8 x, int i, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
  const b2 v = {x[2 * i], x[2 * i + 1]};
  return __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
}

// LDS writes of a wave must land before its reads of them, and its reads before
// its next writes: LDS executes one wave's operations in order, so only the
// compiler must be kept from moving them across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Compile-time LDS stage index passed to generic lambdas.
template <int N> struct Stage { static constexpr int value = N; };

// Workgroup ids are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical ids so the query tiles of one head share that
// XCD's L2 (and their K/V reads hit it).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3;
  if (bid >= (per << 3)) return bid;
  return (bid & 7) * per + (bid >> 3);
}

// Work order without a band: the (batch, head) pairs are dealt out round-robin
// over the 8 XCDs (pair p runs on XCD p mod 8, since workgroup ids go to the
// XCDs round-robin) and each pair's tiles stay on its XCD, where they share the
// pair's K/V in L2. Every XCD gets every eighth pair, so packed sequences of
// unequal length still spread evenly over the XCDs (contiguous ranges of pairs
// per XCD gave one XCD 1.7x the mean work on a 16-sequence batch). Falls back
// to contiguous ranges when the pair count is not a multiple of 8. With
// grouped-query heads (`group` consecutive query heads per KV head) the pairs
// of one KV head all go to the same XCD, where they share its K/V.
__device__ __forceinline__ void xcd_heads(int bid, int ntiles, int nheads, int n, int& tile, int& head,
                                          int group = 1) {
  if ((nheads & 7) == 0) {
    const int m = bid >> 3;
    const int hl = m / ntiles;
    tile = m - hl * ntiles;
    const int x = bid & 7;
    head = (group > 1 && nheads % (8 * group) == 0) ? (x + 8 * (hl / group)) * group + hl % group
                                                   : hl * 8 + x;
  } else {
    const int r = xcd_remap(bid, n);
    tile = r % ntiles;
    head = r / ntiles;
  }
}

// Work order for masks that make tile workloads uneven (causal). Workgroup ids
// go to the heads in blocks of hb heads (the host sizes a block so that its
// operands stay resident in the last-level cache); inside a block the tiles
// come heaviest first, with the head varying fastest, so the ids on one XCD
// (id mod 8) keep revisiting the same heads and the machine drains on light
// tiles. `order` 0 is the heaviest tile; the caller maps it to a tile index.
// With grouped-query heads (`group` query heads per KV head, consecutive), the
// heads inside a block are permuted so that all query heads of one KV head
// land on the same XCD and share its K/V in that XCD's L2 (when the block size
// is a multiple of 8 groups; otherwise the plain order).
__device__ __forceinline__ void blocked_order(int p, int ntiles, int nheads, int hb, int& order, int& head,
                                              int group = 1) {
  const int per_block = hb * ntiles;
  const int blk = p / per_block;
  const int r = p - blk * per_block;
  const int cnt = min(hb, nheads - blk * hb);
  order = r / cnt;
  int hi = r - order * cnt;   // slot in the block: XCD = hi mod 8
  if (group > 1 && hb % group == 0 && cnt % (8 * group) == 0) {
    const int x = hi & 7, t = hi >> 3;
    hi = (x + 8 * (t / group)) * group + t % group;
  }
  head = blk * hb + hi;
}

}  // namespace fa
