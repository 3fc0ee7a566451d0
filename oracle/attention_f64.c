/*
 * Oracle for exact attention: plain fp64 CPU code.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do. It shares no code with the HIP kernels.
 *
 * What it computes is the definition printed in the "flash-attention-v100"
 * README (section "How to use FlashAttention"): O = softmax(scale * Q K^T) V,
 * with
 *   - the grouped-query head map of the flash_attn_func docstring: query head
 *     h reads key/value head h / (Hq / Hkv) (6 query heads over 2 KV heads:
 *     heads 0-2 use KV head 0, heads 3-5 use KV head 1);
 *   - the causal mask aligned to the bottom-right corner (Changelog 2.1 and the
 *     flash_attn_with_kvcache docstring): query i may see key j iff
 *     j <= i + Nk - Nq; a row with no visible key gives an all-zero output;
 *   - the sliding-window band of the same docstrings: keys in
 *     [i + Nk - Nq - left, i + Nk - Nq + right], a negative bound meaning
 *     unbounded;
 *   - the per-sequence key length (cache_seqlens) of flash_attn_with_kvcache:
 *     batch b uses Nk_b = seqlens_k[b] keys when seqlens_k is given;
 *   - an optional key range [key_begin, key_end) so the same routine yields the
 *     per-chunk results of the Flash-Decoding steps ("flash attention-2 github"
 *     search page, Flash-Decoding description).
 *
 * It also returns the per-row log-sum-exp of the scaled, masked scores
 * (natural log), the scalar that Flash-Decoding writes per row and per split.
 * A row with no visible key gets LSE = -infinity.
 *
 * Method: two passes per row over the stored scores (exact maximum first, then
 * exponentials and sums), in double precision, with OpenMP over
 * (batch, head, query row), the sequence-of-Q partition the "Flash attention
 * gpu" page mentions for its CPU version. No tiling, no online softmax.
 *
 * Layouts: q [B][Nq][Hq][d], k and v [B][Nk][Hkv][d], o [B][Nq][Hq][d] and
 * lse [B][Hq][Nq], all row-major doubles.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>

static int visible(long i, long j, long nq, long nk, int causal, long wl, long wr,
                   long kb, long ke) {
  long diag = i + nk - nq;
  if (j < kb || j >= ke || j >= nk) return 0;
  if (causal && j > diag) return 0;
  if (wl >= 0 && j < diag - wl) return 0;
  if (wr >= 0 && j > diag + wr) return 0;
  return 1;
}

/* Returns 0 on success, 1 on bad arguments, 2 when out of memory. */
int oracle_attention_f64(const double* q, const double* k, const double* v,
                         double* o, double* lse,
                         long B, long Nq, long Nk, long Hq, long Hkv, long d,
                         int causal, long window_left, long window_right,
                         const int* seqlens_k, long key_begin, long key_end,
                         double scale) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv != 0)
    return 1;
  long group = Hq / Hkv;
  int failed = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!s || !acc) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for collapse(3) schedule(dynamic, 1)
    for (long b = 0; b < B; b++)
      for (long h = 0; h < Hq; h++)
        for (long i = 0; i < Nq; i++) {
          if (!s || !acc) continue;
          long g = h / group;
          long nk = seqlens_k ? (long)seqlens_k[b] : Nk;
          if (nk > Nk) nk = Nk;
          const double* qi = q + ((b * Nq + i) * Hq + h) * d;
          double* oi = o + ((b * Nq + i) * Hq + h) * d;
          /* pass 1: scores of the visible keys and their exact maximum */
          double m = -INFINITY;
          long cnt = 0;
          for (long j = 0; j < nk; j++) {
            if (!visible(i, j, Nq, nk, causal, window_left, window_right, key_begin, key_end))
              continue;
            const double* kj = k + ((b * Nk + j) * Hkv + g) * d;
            double dot = 0.0;
            for (long c = 0; c < d; c++) dot += qi[c] * kj[c];
            s[j] = scale * dot;
            if (s[j] > m) m = s[j];
            cnt++;
          }
          if (cnt == 0) {
            for (long c = 0; c < d; c++) oi[c] = 0.0;
            lse[(b * Hq + h) * Nq + i] = -INFINITY;
            continue;
          }
          /* pass 2: exponentials, their sum, and the weighted sum of V rows */
          double l = 0.0;
          for (long c = 0; c < d; c++) acc[c] = 0.0;
          for (long j = 0; j < nk; j++) {
            if (!visible(i, j, Nq, nk, causal, window_left, window_right, key_begin, key_end))
              continue;
            double p = exp(s[j] - m);
            l += p;
            const double* vj = v + ((b * Nk + j) * Hkv + g) * d;
            for (long c = 0; c < d; c++) acc[c] += p * vj[c];
          }
          for (long c = 0; c < d; c++) oi[c] = acc[c] / l;
          lse[(b * Hq + h) * Nq + i] = m + log(l);
        }
    free(s);
    free(acc);
  }
  return failed ? 2 : 0;
}

/* Number of threads the OpenMP runtime will use (for reporting). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}
