// Host-side launch interface between the C ABI (fa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  int B, Nq, Nk, Hq, Hkv;
  int group;       // Hq / Hkv
  int n_qtiles;    // ceil(Nq / rows per workgroup)
  float sl2;       // |scale| * log2(e)
  int negate_q;    // scale < 0: the kernel flips the sign of Q instead
  // band of visible keys for query i (diag = Nk - Nq): i + diag - wl <= j <= i + diag + wr;
  // -1 leaves that side open. Causal is wl = -1, wr = 0.
  int wl, wr;
  // packed variable-length batch (cu_q non-null): q/o are [total_q][Hq][d], k/v
  // [total_k][Hkv][d], lse [Hq][total_q]; sequence b owns rows cu_q[b] ..
  // cu_q[b+1] of q and cu_k[b] .. cu_k[b+1] of k; Nq is the longest query count
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int hb;          // heads per block of the heaviest-first order used with a band
  int wide;        // d = 128 fp16 without a band: eight-wave workgroups of 256 rows
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null
  float* part_o;   // [S][B][Hq][Nq][d] float32
  float* part_lse; // [S][B][Hq][Nq] float32, log2 domain
  int B, Nq, Nk, Hq, Hkv;
  int group;       // Hq / Hkv
  int splits;      // parts (partials per row): sub_per parts per requested split
  int sub_per;     // parts per requested split: 1, 2 or 4
  int row_blocks;  // ceil(group * Nq / 32)
  float sl2;       // |scale| * log2(e)
  int negate_q;    // scale < 0: the kernel flips the sign of q instead
  // paged cache (block_table non-null): k and v point at page pools
  // [num_pages][page_size][Hkv][d]; sequence b owns pages block_table[b][0..max_pages)
  // and seqlens[b] keys. For a contiguous cache block_table and seqlens are null.
  const int* block_table;
  const int* seqlens;
  int page_size, max_pages, num_pages;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;  // [B][Hq][Nq], natural log, from the forward pass
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;       // workspace [B][Hq][Nq rounded up to 32]: sum_c dO * O
  float* lse2;       // workspace, same shape: LSE * log2(e), +inf for no key / padding
  int B, Nq, Nk, Hq, Hkv;
  int group;         // Hq / Hkv
  float sl2;         // scale * log2(e)
  float scale;
  // band of visible keys for query i (diag = Nk - Nq): i + diag - wl <= j <= i + diag + wr;
  // -1 leaves that side open. Causal is wl = -1, wr = 0.
  int wl, wr;
  int hb_kv, hb_q;   // heads per block of the heaviest-first causal orders (dK/dV, dQ)
  // packed variable-length batch (cu_q non-null): q/o/dout/dq are [total_q][Hq][d],
  // k/v/dk/dv [total_k][Hkv][d], lse [Hq][total_q]; sequence b owns rows
  // cu_q[b] .. cu_q[b+1] and cu_k[b] .. cu_k[b+1]; Nq, Nk are the longest counts
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
};

// Heads per block for blocked_order: as many (batch, head) pairs as keep
// `bytes_per_head` of operands within 64 MiB, a multiple of 8 (one per XCD) when
// there are at least 8.
inline int order_block_heads(long long nheads, long long bytes_per_head) {
  long long hb = (64ll << 20) / (bytes_per_head > 0 ? bytes_per_head : 1);
  hb = hb < 8 ? 8 : hb / 8 * 8;
  return static_cast<int>(hb < nheads ? hb : nheads);
}

// Rows of queries one forward workgroup covers (32 per wave).
constexpr int fwd_rows(int, bool wide = false) { return wide ? 256 : 128; }

// band: apply the (wl, wr) band (causal or a sliding window)
hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool band, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, bool causal, hipStream_t stream);
// band: apply the (wl, wr) band (causal or a sliding window)
hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool band, hipStream_t stream);

}  // namespace fa
