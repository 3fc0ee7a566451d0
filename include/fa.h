/*
 * fa.h -- C ABI of libfa: exact tiled attention on MI355X (gfx950).
 *
 * Three operations:
 *   fa_fwd             the exact attention forward pass, computed tile by tile
 *                      with an online softmax so the Nq x Nk score matrix never
 *                      reaches device memory (variants: fa_fwd_window,
 *                      fa_fwd_varlen);
 *   fa_decode_splitkv  the same result for short query blocks, with the keys
 *                      split into parts that are processed in parallel and a
 *                      second kernel that merges the per-part results
 *                      (variant: fa_decode_splitkv_paged);
 *   fa_bwd             the gradients dQ, dK, dV of the forward pass, again
 *                      without storing the score matrix.
 *
 * Definition ("flash-attention-v100" README, How to use FlashAttention):
 *   O = softmax(scale * Q K^T) V, row by row, with
 *   - grouped-query heads: query head h reads key/value head h / (Hq / Hkv);
 *     Hq must be a multiple of Hkv (flash_attn_func docstring);
 *   - causal = 1: query i sees key j iff j <= i + Nk - Nq, the mask aligned to
 *     the bottom-right corner (Changelog 2.1; flash_attn_with_kvcache
 *     docstring); a row that sees no key gets O = 0.
 * Flash-Decoding ("flash attention-2 github" search page; "flash-attention-v100"
 * README, Changelog 2.2): split the keys into parts, attend to each part in
 * parallel while writing one log-sum-exp per row and part, then combine.
 *
 * Layouts (row-major, head_dim fastest; "ampere_flash_attention_from_scratch"
 * README, Performance Test header [batch_size, seq_len, num_heads, head_dim]):
 *   q, o      [B][Nq][Hq][d]   dtype
 *   k, v      [B][Nk][Hkv][d]  dtype  (for decode: the KV cache)
 *   lse       [B][Hq][Nq]      float32, natural log of sum_j exp(scale*q.k_j)
 *                              over the visible keys; -inf for a row that sees
 *                              no key. May be NULL (then not written).
 *
 * Ownership and execution: every pointer is a device pointer owned by the
 * caller. The library never allocates, frees or synchronises; it enqueues
 * kernels on `stream` (a hipStream_t; NULL is the default stream) and returns.
 * Calls are stateless and reentrant. Outputs are fully overwritten.
 *
 * Errors: arguments are validated before any HIP call, so a bad call returns a
 * status without touching the GPU. FA_ERR_LAUNCH reports a failed launch;
 * faults during execution surface at the caller's next synchronisation.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULLPTR = 1,   /* a required pointer is NULL                       */
  FA_ERR_SHAPE = 2,     /* B, Nq, Nk, Hq or Hkv < 1, or a size overflows    */
  FA_ERR_HEADS = 3,     /* Hq is not a multiple of Hkv                      */
  FA_ERR_HEADDIM = 4,   /* d not in {32, 64, 96, 128, 192, 256}             */
  FA_ERR_DTYPE = 5,     /* dtype not FA_F16 or FA_BF16                      */
  FA_ERR_SPLITS = 6,    /* num_splits < 1 or > FA_MAX_SPLITS                */
  FA_ERR_WORKSPACE = 7, /* workspace_bytes below the *_workspace_bytes size  */
  FA_ERR_LAUNCH = 8,    /* the HIP runtime rejected a kernel launch         */
  FA_ERR_ALIGN = 9,     /* a tensor pointer is not 16-byte aligned          */
  FA_ERR_SCALE = 10,    /* scale is not a finite number                     */
  FA_ERR_SCRATCH = 11   /* the call needs more than the fixed scratch holds  */
} fa_status;

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

#define FA_MAX_SPLITS 256

/*
 * Attention forward pass.
 *   q, k, v, o : device tensors in the layouts above, `dtype` elements,
 *                16-byte aligned. o must not overlap q, k or v.
 *   lse        : device float32 [B][Hq][Nq] or NULL.
 *   B, Nq, Nk, Hq, Hkv, d : sizes; Nq != Nk is allowed (with causal = 1 the
 *                mask is bottom-right aligned). FA_ERR_SHAPE when a tensor
 *                holds more than 2^40 elements, Hq * d exceeds 2^22, or one
 *                of the call's kernel grids would exceed 2^32 - 1 threads
 *                (the same limits hold for every entry point below).
 *   causal     : 0 or 1 (any non-zero value means 1).
 *   scale      : multiplies Q K^T before the softmax, used exactly as passed
 *                (the pages' default is 1/sqrt(d); the Python layer applies it).
 *   dtype      : FA_F16 or FA_BF16; accumulation is float32, P is rounded to
 *                dtype before the P V product, O is rounded to nearest even.
 * Returns FA_OK or an error status; on error nothing is enqueued.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Nq, int Nk, int Hq, int Hkv, int d, int causal, float scale,
                 fa_dtype dtype, void* stream);

/*
 * Attention forward pass with a sliding window (local attention;
 * "flash-attention-v100" README, How to use FlashAttention: window_size, and
 * Changelog 2.3): query i sees key j iff
 *   i + Nk - Nq - window_left <= j <= i + Nk - Nq + window_right,
 * the band aligned to the bottom-right corner like the causal mask; -1 leaves
 * a side unbounded. causal = 1 sets window_right to 0. A row that sees no key
 * gets O = 0 and LSE = -inf. fa_fwd is this call with window (-1, -1).
 * Other arguments, layouts and status codes as in fa_fwd; FA_ERR_SHAPE for a
 * window side below -1.
 */
fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Nq, int Nk, int Hq, int Hkv, int d, int window_left,
                        int window_right, int causal, float scale, fa_dtype dtype, void* stream);

/*
 * Attention forward pass over a packed batch of variable-length sequences (the
 * flash_attn_varlen_func entry point named in the "flash-attention-v100"
 * README, Changelog 2.0; the argument reading is ours): sequence b owns query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1, and attends only within itself.
 *   q, o          : [total_q][Hq][d]; k, v: [total_k][Hkv][d]; all `dtype`.
 *   lse           : float32 [Hq][total_q] or NULL.
 *   cu_seqlens_q,
 *   cu_seqlens_k  : device int32 [B + 1], non-decreasing prefix sums starting
 *                   at 0 and ending at total_q / total_k. Values are clamped to
 *                   [0, total]; a malformed table gives undefined results for
 *                   the affected sequences but no access outside the tensors.
 *   max_seqlen_q  : at least the longest query count (it sizes the grid; rows
 *                   beyond a sequence's own count are not computed). A value
 *                   below some sequence's query count leaves that sequence's
 *                   rows from ceil(max_seqlen_q / 128) * 128 on unwritten (no
 *                   access outside the tensors); the Python binding checks it.
 *   causal        : bottom-right aligned per sequence, as in fa_fwd. A
 *                   sequence with no key gets O = 0 and LSE = -inf.
 * Status: FA_ERR_NULLPTR for a NULL prefix-sum array, FA_ERR_ALIGN for a
 * misaligned one, FA_ERR_SHAPE for B or max_seqlen_q < 1 or totals < 1,
 * otherwise as fa_fwd.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                        int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                        fa_dtype dtype, void* stream);

/*
 * Bytes of device workspace fa_decode_splitkv needs. Each of the num_splits
 * splits is processed as up to 4 parts with a partial result each; the
 * workspace holds float32 partial outputs [4*num_splits][B][Hq][Nq][d]
 * followed by float32 partial LSEs [4*num_splits][B][Hq][Nq], each part
 * padded to 256 bytes. Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits);

/*
 * Split-KV attention (Flash-Decoding) over a contiguous KV cache.
 *   q, o       : [B][Nq][Hq][d]; k_cache, v_cache: [B][Nk][Hkv][d]; all `dtype`.
 *   lse        : float32 [B][Hq][Nq] or NULL.
 *   num_splits : number of key splits S, 1..FA_MAX_SPLITS. The keys are cut
 *                into 32-key tiles; each split is processed as P = 1, 2 or 4
 *                parts (P grows when there are few splits x heads x batch),
 *                and part p of the P*S parts takes tiles p, p + P*S,
 *                p + 2*P*S, ... (tile-interleaved, so the parts read
 *                neighbouring tiles at the same time). Parts with no tile are
 *                empty and weigh nothing. The merged result does not depend on
 *                the partition beyond float32 rounding.
 *                Nk * Hkv * d * 2 must stay below 2^31, and Hkv times
 *                ceil(Hq / Hkv * Nq / 32) at most 65535 (FA_ERR_SHAPE).
 *   causal     : as in fa_fwd (bottom-right aligned against Nk).
 *   workspace  : caller-owned device buffer of at least
 *                fa_decode_workspace_bytes(B, Nq, Hq, d, num_splits) bytes,
 *                16-byte aligned; its contents on entry do not matter.
 * Two kernels are enqueued on `stream`: the per-part pass, then the merge.
 * The result equals fa_fwd's on the same inputs up to float32 rounding.
 */
fa_status fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o,
                            float* lse, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                            int num_splits, int causal, float scale, fa_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_splitkv for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and the same result, bit for bit, with
 * the per-part partials in a fixed device array of FA_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU until the process ends. No allocation,
 * free or allocating library routine is called.
 *   Arguments, layouts and status codes as fa_decode_splitkv without the
 *   workspace. FA_ERR_SCRATCH (before any HIP call) when the call's partials,
 *   float32 [P*S][B][Hq][Nq][d] and [P*S][B][Hq][Nq] each padded to 256 bytes
 *   (P parts per split as described there), exceed FA_NOALLOC_SCRATCH_BYTES;
 *   the decode workloads B=8, Nq=1 and 8, Nk=8192, Hq=32, Hkv=8, d=128, S=16
 *   take about 2 and 16 MiB. FA_ERR_LAUNCH if the array's address cannot be found.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (on different streams, or from different threads) race and give undefined
 * results; calls ordered on one stream are fine. Its contents on entry do not
 * matter (every part writes its partial before the merge reads it).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                    float* lse, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                                    int num_splits, int causal, float scale, fa_dtype dtype, void* stream);

/*
 * Split-KV attention over a paged KV cache with per-sequence lengths
 * ("flash-attention-v100" README, How to use FlashAttention: the block_table and
 * cache_seqlens arguments of flash_attn_with_kvcache).
 *   q, o          : [B][Nq][Hq][d], `dtype`; lse: float32 [B][Hq][Nq] or NULL.
 *   k_pages,
 *   v_pages       : page pools [num_pages][page_size][Hkv][d], `dtype`.
 *   block_table   : device int32 [B][max_pages_per_seq]; key j of sequence b
 *                   lives in page block_table[b][j / page_size], row
 *                   j % page_size. Entries past the sequence's last page are
 *                   not read. An entry outside [0, num_pages) makes its keys
 *                   read as zero vectors (results for that sequence are then
 *                   undefined, but no memory outside the pools is touched).
 *   cache_seqlens : device int32 [B]; sequence b has cache_seqlens[b] keys,
 *                   clamped to [0, max_pages_per_seq * page_size]. A sequence
 *                   with no key gets O = 0 and LSE = -inf.
 *   page_size     : a multiple of 32 (>= 32).
 *   num_splits    : as in fa_decode_splitkv; the tiles of sequence b are those
 *                   below its own length.
 *   causal        : bottom-right aligned against each sequence's length.
 *   workspace     : fa_decode_workspace_bytes(B, Nq, Hq, d, num_splits) bytes.
 * A contiguous cache [B][Nk][Hkv][d] with per-sequence lengths is the special
 * case page_size = Nk (a multiple of 32), num_pages = B, block_table[b] = {b}.
 * Status: FA_ERR_NULLPTR for a NULL block_table or cache_seqlens,
 * FA_ERR_SHAPE for a bad page geometry, FA_ERR_ALIGN for a misaligned int32
 * array, otherwise as fa_decode_splitkv.
 */
fa_status fa_decode_splitkv_paged(const void* q, const void* k_pages, const void* v_pages,
                                  const int* block_table, const int* cache_seqlens, void* o,
                                  float* lse, int B, int Nq, int Hq, int Hkv, int d, int num_pages,
                                  int page_size, int max_pages_per_seq, int num_splits, int causal,
                                  float scale, fa_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace fa_bwd needs: two float32 arrays [B][Hq][Nq'] with
 * Nq' = Nq rounded up to a multiple of 64, each padded to 256 bytes. Returns 0
 * for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int Nq, int Hq);

/*
 * Attention backward pass ("flash-attention-v100" README: the package's
 * backward pass and its deterministic option; Changelog 2.1 for the
 * bottom-right causal mask it shares with the forward). With P the softmax
 * probabilities of the forward pass and D_i = sum_c dO[i][c] O[i][c]:
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
 * where for grouped-query heads dK and dV of a KV head sum over the query
 * heads that read it. P is recomputed from `lse`, never stored.
 *   q, k, v, o : the forward pass's inputs and output (layouts above).
 *   lse        : float32 [B][Hq][Nq], the forward pass's log-sum-exp
 *                (required; -inf marks a row with no visible key).
 *   dout       : dO, [B][Nq][Hq][d] `dtype`.
 *   dq         : [B][Nq][Hq][d]; dk, dv: [B][Nk][Hkv][d]; all `dtype`, fully
 *                overwritten, not overlapping any input or each other.
 *   causal, scale, dtype : as passed to the forward pass.
 *   workspace  : caller-owned device buffer of at least
 *                fa_bwd_workspace_bytes(B, Nq, Hq) bytes, 16-byte aligned; its
 *                contents on entry do not matter.
 * Accumulation is float32; P and dS are rounded to dtype as MFMA operands.
 * There are no atomics: the result is identical from run to run. Three
 * kernels are enqueued on `stream` (row statistics, dK/dV, dQ).
 * Status: FA_ERR_NULLPTR for a NULL lse, dout, dq, dk, dv or workspace,
 * FA_ERR_WORKSPACE for a short workspace, FA_ERR_SHAPE when B * Hq * Nq'
 * exceeds 2^28 - 1, otherwise as fa_fwd.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                 int Hkv, int d, int causal, float scale, fa_dtype dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Attention backward pass with a sliding window: the gradients of
 * fa_fwd_window's result, with the band, its bottom-right alignment, the -1
 * convention and causal fixing window_right = 0 as there. fa_bwd is this call
 * with window (-1, -1). Other arguments, layouts and status codes as in
 * fa_bwd; FA_ERR_SHAPE for a window side below -1.
 */
fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int B, int Nq, int Nk, int Hq,
                        int Hkv, int d, int window_left, int window_right, int causal, float scale,
                        fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention backward pass over a packed batch of variable-length sequences:
 * the gradients of fa_fwd_varlen's result (same packing, prefix sums and
 * bottom-right causal mask per sequence).
 *   q, o, dout, dq : [total_q][Hq][d]; k, v, dk, dv: [total_k][Hkv][d]; `dtype`.
 *   lse            : float32 [Hq][total_q], as fa_fwd_varlen writes it.
 *   cu_seqlens_q,
 *   cu_seqlens_k   : device int32 [B + 1], as for fa_fwd_varlen.
 *   max_seqlen_q,
 *   max_seqlen_k   : at least every sequence's query / key count (they size the
 *                    grid and the workspace). A smaller value clips the longer
 *                    sequences to their first max_seqlen rows / keys, which moves
 *                    their causal diagonal: their gradients are then those of the
 *                    clipped problem, not of fa_fwd_varlen's result (no access
 *                    outside the tensors or the workspace); the Python binding
 *                    checks the lengths.
 *   workspace      : fa_bwd_workspace_bytes(B, max_seqlen_q, Hq) bytes.
 * Rows of dq, dk, dv outside every sequence are not written. Status:
 * FA_ERR_NULLPTR for a NULL prefix-sum array, FA_ERR_ALIGN for a misaligned one,
 * FA_ERR_SHAPE for B, max_seqlen_q or max_seqlen_k < 1, otherwise as fa_bwd.
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k, int total_q,
                        int total_k, int Hq, int Hkv, int d, int causal, float scale, fa_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_str(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
