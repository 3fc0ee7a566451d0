// C ABI of libfa: argument validation and dispatch. Every check runs before
// the first HIP call, so invalid calls return a status without a GPU.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_fwd_d32(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_fwd_d64(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_fwd_d96(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_fwd_d128(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_fwd_d192(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_fwd_d256(const FwdArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d32(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d64(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d96(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d128(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d192(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_decode_d256(const DecodeArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d32(const BwdArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d64(const BwdArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d96(const BwdArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d128(const BwdArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d192(const BwdArgs&, bool, bool, hipStream_t);
hipError_t launch_bwd_d256(const BwdArgs&, bool, bool, hipStream_t);

hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool band, hipStream_t s) {
  switch (d) {
    case 32: return launch_fwd_d32(a, bf16, band, s);
    case 64: return launch_fwd_d64(a, bf16, band, s);
    case 96: return launch_fwd_d96(a, bf16, band, s);
    case 128: return launch_fwd_d128(a, bf16, band, s);
    case 192: return launch_fwd_d192(a, bf16, band, s);
    case 256: return launch_fwd_d256(a, bf16, band, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, bool causal, hipStream_t s) {
  switch (d) {
    case 32: return launch_decode_d32(a, bf16, causal, s);
    case 64: return launch_decode_d64(a, bf16, causal, s);
    case 96: return launch_decode_d96(a, bf16, causal, s);
    case 128: return launch_decode_d128(a, bf16, causal, s);
    case 192: return launch_decode_d192(a, bf16, causal, s);
    case 256: return launch_decode_d256(a, bf16, causal, s);
  }
  return hipErrorInvalidValue;
}

fa_status noalloc_scratch(void** ptr, size_t* bytes);   // fa_noalloc.hip

hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool band, hipStream_t s) {
  switch (d) {
    case 32: return launch_bwd_d32(a, bf16, band, s);
    case 64: return launch_bwd_d64(a, bf16, band, s);
    case 96: return launch_bwd_d96(a, bf16, band, s);
    case 128: return launch_bwd_d128(a, bf16, band, s);
    case 192: return launch_bwd_d192(a, bf16, band, s);
    case 256: return launch_bwd_d256(a, bf16, band, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace fa

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;  // per tensor, keeps 64-bit offsets far from overflow
// Hq * d at most 2^22 elements: the kernels address a tile of up to 64 rows
// from its first row with 32-bit byte offsets (row x heads x d x 2 bytes), so
// one row of all heads must stay below 2^31 / 64 bytes.
constexpr int64_t kMaxRowElems = int64_t(1) << 22;
// A dispatch counts at most 2^32 - 1 work-items per grid dimension (its size
// field is 32-bit). Every grid here spreads its workgroups along x, with at
// most 256 threads each; checking all of a call's grids before the first launch
// keeps a failed call from leaving part of its kernels enqueued.
constexpr int64_t kMaxGroupsX = 0xffffffffLL / 256;

bool head_dim_ok(int d) {
  return d == 32 || d == 64 || d == 96 || d == 128 || d == 192 || d == 256;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status check_common(const void* q, const void* k, const void* v, void* o, const float* lse,
                       int B, int Nq, int Nk, int Hq, int Hkv, int d, float scale, fa_dtype dtype) {
  if (!q || !k || !v || !o) return FA_ERR_NULLPTR;
  if (B < 1 || Nq < 1 || Nk < 1 || Hq < 1 || Hkv < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_HEADS;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t qe = int64_t(B) * Nq * Hq * d, ke = int64_t(B) * Nk * Hkv * d;
  if (qe > kMaxElems || ke > kMaxElems) return FA_ERR_SHAPE;
  if (int64_t(Hq) * d > kMaxRowElems) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_ALIGN;
  return FA_OK;
}

size_t pad256(size_t x) { return (x + 255) & ~size_t(255); }

// each requested split is processed as up to this many parts, each with its
// own partial (the workspace is sized for the maximum)
constexpr int kSubPerChunk = 4;
// single-wave workgroups that give the chip about one round (256 CUs x 4 SIMDs)
constexpr int64_t kDecodeWaves = 1024;

// Parts per requested split: 1, 2 or 4, so that the split grid has about
// kDecodeWaves single-wave workgroups.
int decode_sub_per(int B, int Nq, int Hq, int Hkv, int num_splits) {
  const int64_t row_blocks = (int64_t(Hq / Hkv) * Nq + 31) / 32;
  const int64_t units = int64_t(num_splits) * Hkv * row_blocks * B;
  return units >= kDecodeWaves ? 1 : (2 * units >= kDecodeWaves ? 2 : kSubPerChunk);
}

// Bytes of partials for `slices` part slices: float32 [slices][B][Hq][Nq][d]
// then float32 [slices][B][Hq][Nq], each padded to 256 bytes.
size_t decode_partial_bytes(int64_t slices, int B, int Nq, int Hq, int d) {
  const size_t rows = size_t(slices) * B * Hq * Nq;
  return pad256(rows * d * sizeof(float)) + pad256(rows * sizeof(float));
}

// Fills the rest of the decode arguments (cache fields already set), checks the
// grid limits and enqueues the split and combine kernels. The workspace holds
// `slices` part slices of partials (at least the parts this call uses).
fa_status launch_decode_common(fa::DecodeArgs& a, const void* q, void* o, float* lse, int B, int Nq,
                               int Hq, int Hkv, int d, int num_splits, int causal, float scale,
                               fa_dtype dtype, void* workspace, int64_t slices, void* stream) {
  const int group = Hq / Hkv;
  const int64_t row_blocks = (int64_t(group) * Nq + 31) / 32;
  // split grid: x = batch, y = parts, z = KV heads x row blocks (y and z at most 65535)
  if (int64_t(kSubPerChunk) * num_splits > 65535 || row_blocks * Hkv > 65535) return FA_ERR_SHAPE;
  // combine grid: B x ceil(Hq * Nq / rows per workgroup), d / 4 threads per row
  const int64_t combine_rows = 1024 / d;
  if (int64_t(B) > kMaxGroupsX || int64_t(B) * ((int64_t(Hq) * Nq + combine_rows - 1) / combine_rows) > kMaxGroupsX)
    return FA_ERR_SHAPE;
  a.q = q; a.o = o; a.lse = lse;
  const size_t rows = size_t(slices) * B * Hq * Nq;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pad256(rows * d * sizeof(float)));
  a.B = B; a.Nq = Nq; a.Hq = Hq; a.Hkv = Hkv;
  a.group = group;
  a.sub_per = decode_sub_per(B, Nq, Hq, Hkv, num_splits);
  a.splits = a.sub_per * num_splits;
  a.row_blocks = static_cast<int>(row_blocks);
  // the kernels take the reference max of the raw scores times sl2, which must not
  // be negative: a negative scale is applied by flipping the sign of q (exact)
  a.sl2 = fabsf(scale) * 1.4426950408889634f;
  a.negate_q = scale < 0.f;
  hipError_t e = fa::launch_decode(a, d, dtype == FA_BF16, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Fills the rest of the forward arguments (tensors and sizes already set) and
// enqueues the kernel. Causal fixes the right edge of the band at the diagonal.
fa_status fwd_common(fa::FwdArgs& a, int d, int wl, int wr, int causal, float scale, fa_dtype dtype,
                     void* stream) {
  a.group = a.Hq / a.Hkv;
  a.sl2 = fabsf(scale) * 1.4426950408889634f;
  a.negate_q = scale < 0.f;
  a.wl = wl;
  a.wr = causal ? 0 : wr;
  const int64_t blocks = int64_t((a.Nq + fa::fwd_rows(d) - 1) / fa::fwd_rows(d)) * a.Hq * a.B;
  if (blocks > kMaxGroupsX) return FA_ERR_SHAPE;
  // long fp16 sequences at d = 128 without a band take the eight-wave shape:
  // at 3072 rows and more it measured 3-4% faster, shorter ones and bf16 (whose
  // extra row sum wants the third wave per SIMD) gain nothing from it
  a.wide = d == 128 && dtype == FA_F16 && a.wl < 0 && a.wr < 0 && a.cu_q == nullptr && a.Nq >= 3072;
  // its workgroups have 512 threads: keep the dispatch within 2^32 - 1 of them
  if (a.wide && int64_t((a.Nq + fa::fwd_rows(d, true) - 1) / fa::fwd_rows(d, true)) * a.Hq * a.B > kMaxGroupsX / 2)
    a.wide = 0;
  a.n_qtiles = (a.Nq + fa::fwd_rows(d, a.wide) - 1) / fa::fwd_rows(d, a.wide);
  // K and V bytes each query head reads (a group shares them)
  const int64_t kv_rows = a.cu_k ? int64_t(a.total_k) / a.B : a.Nk;
  a.hb = fa::order_block_heads(int64_t(a.Hq) * a.B, kv_rows * d * 4 / a.group);
  const bool band = a.wl >= 0 || a.wr >= 0;
  hipError_t e = fa::launch_fwd(a, d, dtype == FA_BF16, band, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// rows of each backward statistics array: [B][Hq][Nq rounded up to 64]
size_t bwd_stat_rows(int B, int Nq, int Hq) { return size_t(B) * Hq * ((size_t(Nq) + 63) / 64 * 64); }

fa_status bwd_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, const int* cu_q, const int* cu_k,
                     int total_q, int total_k, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                     int window_left, int window_right, int causal, float scale, fa_dtype dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULLPTR;
  if (window_left < -1 || window_right < -1) return FA_ERR_SHAPE;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, Nq, Hq)) return FA_ERR_WORKSPACE;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_ALIGN;
  const int64_t nkt = (int64_t(Nk) + 127) / 128, nqt = (int64_t(Nq) + 127) / 128;
  if (nkt * Hkv * B > kMaxGroupsX || nqt * Hq * B > kMaxGroupsX) return FA_ERR_SHAPE;
  // the statistics kernel gives a row up to 32 threads (at least 8 rows per
  // workgroup); this also keeps the arrays' 32-bit byte offsets in range
  if ((bwd_stat_rows(B, Nq, Hq) + 7) / 8 > size_t(kMaxGroupsX)) return FA_ERR_SHAPE;
  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  const size_t rows = bwd_stat_rows(B, Nq, Hq);
  a.dsum = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + pad256(rows * sizeof(float)));
  a.B = B; a.Nq = Nq; a.Nk = Nk; a.Hq = Hq; a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.sl2 = scale * 1.4426950408889634f;
  a.scale = scale;
  a.cu_q = cu_q; a.cu_k = cu_k; a.total_q = total_q; a.total_k = total_k;
  a.wl = window_left;
  a.wr = causal ? 0 : window_right;
  a.hb_kv = fa::order_block_heads(int64_t(Hkv) * B, int64_t(a.group) * Nq * d * 4);   // Q and dO of a group
  a.hb_q = fa::order_block_heads(int64_t(Hq) * B, int64_t(Nk) * d * 4 / a.group);     // K and V per query head
  const bool band = a.wl >= 0 || a.wr >= 0;
  hipError_t e = fa::launch_bwd(a, d, dtype == FA_BF16, band, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                 fa_dtype dtype, void* stream) {
  return fa_fwd_window(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, -1, -1, causal, scale, dtype, stream);
}

fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Nq, int Nk, int Hq, int Hkv, int d, int window_left,
                        int window_right, int causal, float scale, fa_dtype dtype, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Nq, Nk, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (window_left < -1 || window_right < -1) return FA_ERR_SHAPE;
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Nq = Nq; a.Nk = Nk; a.Hq = Hq; a.Hkv = Hkv;
  a.cu_q = nullptr; a.cu_k = nullptr; a.total_q = 0; a.total_k = 0;
  return fwd_common(a, d, window_left, window_right, causal, scale, dtype, stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                        int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                        fa_dtype dtype, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULLPTR;
  // the common checks, with the packed tensors as one batch element of total rows
  fa_status st = check_common(q, k, v, o, lse, 1, total_q, total_k, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 1 || max_seqlen_q < 1) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Nq = max_seqlen_q; a.Nk = total_k; a.Hq = Hq; a.Hkv = Hkv;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.total_q = total_q; a.total_k = total_k;
  return fwd_common(a, d, -1, -1, causal, scale, dtype, stream);
}

size_t fa_decode_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits) {
  if (B < 1 || Nq < 1 || Hq < 1 || !head_dim_ok(d) || num_splits < 1 || num_splits > FA_MAX_SPLITS)
    return 0;
  return decode_partial_bytes(int64_t(kSubPerChunk) * num_splits, B, Nq, Hq, d);
}

fa_status fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o,
                            float* lse, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                            int num_splits, int causal, float scale, fa_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(q, k_cache, v_cache, o, lse, B, Nq, Nk, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!workspace) return FA_ERR_NULLPTR;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  const size_t need = fa_decode_workspace_bytes(B, Nq, Hq, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (int64_t(Nk) * Hkv * d * 2 > 0x7fffffffLL) return FA_ERR_SHAPE;   // 32-bit buffer offsets
  fa::DecodeArgs a;
  a.k = k_cache; a.v = v_cache;
  a.Nk = Nk;
  a.block_table = nullptr; a.seqlens = nullptr;
  a.page_size = 0; a.max_pages = 0; a.num_pages = 0;
  return launch_decode_common(a, q, o, lse, B, Nq, Hq, Hkv, d, num_splits, causal, scale, dtype,
                              workspace, int64_t(kSubPerChunk) * num_splits, stream);
}

fa_status fa_decode_splitkv_paged(const void* q, const void* k_pages, const void* v_pages,
                                  const int* block_table, const int* cache_seqlens, void* o,
                                  float* lse, int B, int Nq, int Hq, int Hkv, int d, int num_pages,
                                  int page_size, int max_pages_per_seq, int num_splits, int causal,
                                  float scale, fa_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!block_table || !cache_seqlens) return FA_ERR_NULLPTR;
  if (num_pages < 1 || page_size < 32 || page_size % 32 != 0 || max_pages_per_seq < 1)
    return FA_ERR_SHAPE;
  const int64_t max_keys = int64_t(max_pages_per_seq) * page_size;
  if (max_keys > 0x7fffffffLL) return FA_ERR_SHAPE;
  // the common checks, with the pool standing in for the cache ([1][pool rows][Hkv][d])
  const int64_t pool_rows = int64_t(num_pages) * page_size;
  if (pool_rows > 0x7fffffffLL) return FA_ERR_SHAPE;
  fa_status st = check_common(q, k_pages, v_pages, o, lse, B, Nq, static_cast<int>(pool_rows), Hq, Hkv,
                              d, scale, dtype);
  if (st != FA_OK) return st;
  if (!workspace) return FA_ERR_NULLPTR;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (workspace_bytes < fa_decode_workspace_bytes(B, Nq, Hq, d, num_splits)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(cache_seqlens) & 3u))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a;
  a.k = k_pages; a.v = v_pages;
  a.Nk = static_cast<int>(max_keys);
  a.block_table = block_table; a.seqlens = cache_seqlens;
  a.page_size = page_size; a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  return launch_decode_common(a, q, o, lse, B, Nq, Hq, Hkv, d, num_splits, causal, scale, dtype,
                              workspace, int64_t(kSubPerChunk) * num_splits, stream);
}

fa_status fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                    float* lse, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                                    int num_splits, int causal, float scale, fa_dtype dtype, void* stream) {
  // fa_decode_splitkv's checks, in its order, with the fixed scratch in place of
  // the workspace; the size check comes before the first HIP call
  fa_status st = check_common(q, k_cache, v_cache, o, lse, B, Nq, Nk, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (int64_t(Nk) * Hkv * d * 2 > 0x7fffffffLL) return FA_ERR_SHAPE;   // 32-bit buffer offsets
  // only the parts this call uses: the scratch layout follows the call
  const int64_t slices = int64_t(decode_sub_per(B, Nq, Hq, Hkv, num_splits)) * num_splits;
  if (decode_partial_bytes(slices, B, Nq, Hq, d) > size_t(FA_NOALLOC_SCRATCH_BYTES)) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  st = fa::noalloc_scratch(&ws, &ws_bytes);
  if (st != FA_OK) return st;
  if (decode_partial_bytes(slices, B, Nq, Hq, d) > ws_bytes) return FA_ERR_SCRATCH;
  fa::DecodeArgs a;
  a.k = k_cache; a.v = v_cache;
  a.Nk = Nk;
  a.block_table = nullptr; a.seqlens = nullptr;
  a.page_size = 0; a.max_pages = 0; a.num_pages = 0;
  return launch_decode_common(a, q, o, lse, B, Nq, Hq, Hkv, d, num_splits, causal, scale, dtype, ws, slices,
                              stream);
}

size_t fa_bwd_workspace_bytes(int B, int Nq, int Hq) {
  if (B < 1 || Nq < 1 || Hq < 1) return 0;
  return 2 * pad256(bwd_stat_rows(B, Nq, Hq) * sizeof(float));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                 int Hkv, int d, int causal, float scale, fa_dtype dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return fa_bwd_window(q, k, v, o, lse, dout, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, -1, -1, causal, scale,
                       dtype, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                        int Hkv, int d, int window_left, int window_right, int causal, float scale,
                        fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(q, k, v, const_cast<void*>(o), lse, B, Nq, Nk, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, 0, 0, B, Nq, Nk, Hq, Hkv, d,
                    window_left, window_right, causal, scale, dtype, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k, int total_q,
                        int total_k, int Hq, int Hkv, int d, int causal, float scale, fa_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULLPTR;
  // the common checks, with the packed tensors as one batch element of total rows
  fa_status st = check_common(q, k, v, const_cast<void*>(o), lse, 1, total_q, total_k, Hq, Hkv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (B < 1 || max_seqlen_q < 1 || max_seqlen_k < 1) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, total_q, total_k, B,
                    max_seqlen_q, max_seqlen_k, Hq, Hkv, d, -1, -1, causal, scale, dtype, workspace,
                    workspace_bytes, stream);
}



const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "a size is < 1 or too large";
    case FA_ERR_HEADS: return "Hq is not a multiple of Hkv";
    case FA_ERR_HEADDIM: return "head dim must be one of 32, 64, 96, 128, 192, 256";
    case FA_ERR_DTYPE: return "dtype must be FA_F16 or FA_BF16";
    case FA_ERR_SPLITS: return "num_splits must be in 1..FA_MAX_SPLITS";
    case FA_ERR_WORKSPACE: return "workspace smaller than the size its *_workspace_bytes() call gives";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "scale is not finite";
    case FA_ERR_SCRATCH: return "the call needs more than the FA_NOALLOC_SCRATCH_BYTES of fixed scratch";
  }
  return "unknown status";
}

}  // extern "C"
