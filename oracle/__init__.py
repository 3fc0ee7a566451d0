"""Oracle for exact attention (fp64, CPU).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library and its Python
binding never do. It shares no code with the HIP kernels.

Contents
  attention()        fp64 attention by its definition, in C with OpenMP
                     (attention_f64.c), for any shape
  backward()         fp64 gradients of that definition (dQ, dK, dV for an
                     upstream dO), written out with numpy matrix products
  backward_magnitudes()  per gradient element, the sum of the magnitudes of
                     the terms it adds up (the scale of its rounding error)
  backward_operand_sums()  per gradient element, the sum of the magnitudes of
                     the factors P and dS are multiplied by (the scale of the
                     error of rounding P and dS below the normal range)
  mask_matrix()      the visibility rule of visible() as a boolean matrix
  brute_force()      the same definition as plain Python loops with math.fsum,
                     for tiny shapes; it cross-checks the C routine
  combine_splits()   the third Flash-Decoding step in fp64
  widen()            exact decode of fp16 / bf16 bit patterns to float64

Sources, all restated rather than copied:
  "flash-attention-v100" README, How to use FlashAttention: the definition
  softmax(Q K^T * softmax_scale) V, default scale 1/sqrt(headdim), the GQA head
  map, the bottom-right causal mask with all-zero output for a fully masked
  row, the sliding-window band and cache_seqlens;
  "flash attention-2 github" search page, Flash-Decoding description: split the
  keys/values into chunks, attend to each chunk, write a log-sum-exp per row and
  chunk, then combine.

Where the pages are silent the oracle takes these readings: the LSE is the
natural log-sum-exp of the scaled and masked scores; a row with no visible key
has LSE = -inf; the combine weights chunk s by exp(LSE_s - LSE) with
LSE = log(sum_s exp(LSE_s)), and returns O = 0, LSE = -inf when every chunk is
empty.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_f64.c")
_LIB = os.path.join(_HERE, "liboracle_f64.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain IEEE double arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                               "-shared", "-fPIC", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.oracle_attention_f64.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, L, ctypes.c_int,
                                             L, L, ctypes.POINTER(ctypes.c_int), L, L,
                                             ctypes.c_double]
        lib.oracle_attention_f64.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of 16-bit storage patterns (IEEE binary16 or bfloat16)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def attention(q, k, v, causal=False, scale=None, window=(-1, -1), seqlens_k=None,
              key_range=None):
    """fp64 attention. q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] (float64) -> (o [B,Nq,Hq,d], lse [B,Hq,Nq])."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, Nq, Hq, d), np.float64)
    lse = np.zeros((B, Hq, Nq), np.float64)
    kb, ke = (0, Nk) if key_range is None else key_range
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(seqlens_k, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seqlens_k must have shape (B,)")
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attention_f64(
        q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
        o.ctypes.data_as(dp), lse.ctypes.data_as(dp), B, Nq, Nk, Hq, Hkv, d, int(bool(causal)),
        int(window[0]), int(window[1]),
        None if sl is None else sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
        int(kb), int(ke), float(scale))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, lse


def attention_bits(qb, kb, vb, dtype, **kw):
    """Oracle on 16-bit input patterns, widened exactly to float64."""
    return attention(widen(qb, dtype), widen(kb, dtype), widen(vb, dtype), **kw)


def visible(i, j, Nq, Nk, causal, window=(-1, -1)):
    """Mask predicate, written out for the brute force: may query i see key j?"""
    diag = i + Nk - Nq
    if j < 0 or j >= Nk:
        return False
    if causal and j > diag:
        return False
    if window[0] >= 0 and j < diag - window[0]:
        return False
    if window[1] >= 0 and j > diag + window[1]:
        return False
    return True


def brute_force(q, k, v, causal=False, scale=None, window=(-1, -1), return_probs=False):
    """Pure-Python loops over nested lists/arrays; for tiny shapes only."""
    B, Nq, Hq, d = np.shape(q)
    _, Nk, Hkv, _ = np.shape(k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv
    o = np.zeros((B, Nq, Hq, d))
    lse = np.zeros((B, Hq, Nq))
    probs = np.zeros((B, Hq, Nq, Nk))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Nq):
                keys = [j for j in range(Nk) if visible(i, j, Nq, Nk, causal, window)]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = {j: scale * math.fsum(float(q[b][i][h][c]) * float(k[b][j][g][c])
                                          for c in range(d)) for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                den = math.fsum(e.values())
                for j in keys:
                    probs[b, h, i, j] = e[j] / den
                for c in range(d):
                    o[b, i, h, c] = math.fsum(e[j] * float(v[b][j][g][c]) for j in keys) / den
                lse[b, h, i] = m + math.log(den)
    if return_probs:
        return o, lse, probs
    return o, lse


def combine_splits(o_parts, lse_parts):
    """Merge per-chunk results: o_parts [S,B,Nq,Hq,d], lse_parts [S,B,Hq,Nq] -> (o, lse).

    LSE = log(sum_s exp(LSE_s)); O = sum_s exp(LSE_s - LSE) * O_s. Chunks with
    LSE_s = -inf weigh nothing; if all are -inf the row is O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    mx = np.max(lse_parts, axis=0)
    finite = np.isfinite(mx)
    base = np.where(finite, mx, 0.0)
    w = np.exp(lse_parts - base[None])                     # [S,B,Hq,Nq]
    tot = np.sum(w, axis=0)
    lse = np.where(finite, base + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    o = np.einsum("sbhi,sbihc->bihc", wn, o_parts)
    return o, lse


def mask_matrix(Nq, Nk, causal=False, window=(-1, -1)):
    """Boolean [Nq, Nk]: may query i see key j? The rule of visible(), vectorised."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    diag = i + Nk - Nq
    m = np.ones((Nq, Nk), bool)
    if causal:
        m &= j <= diag
    if window[0] >= 0:
        m &= j >= diag - window[0]
    if window[1] >= 0:
        m &= j <= diag + window[1]
    return m


def backward(q, k, v, do, causal=False, scale=None, window=(-1, -1)):
    """fp64 gradients of L = sum(dO * O) for O = attention(q, k, v): (dq, dk, dv).

    The gradient of the definition, written out (softmax Jacobian):
      P = softmax(scale Q K^T) over the visible keys (0 elsewhere),
      dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
      dQ = scale dS K, dK = scale dS^T Q;
    key/value heads shared by a group of query heads collect the gradients of
    every head of the group. Rows that see no key have P = 0 and contribute
    nothing."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv
    vis = mask_matrix(Nq, Nk, causal, window)
    has = vis.any(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh, kh, vh, doh = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
            s = scale * (qh @ kh.T)
            s = np.where(vis, s, -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            p = e / np.where(has, den, 1.0)[:, None]
            dp = doh @ vh.T
            ds = p * (dp - (p * dp).sum(axis=1)[:, None])
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, g] += scale * (ds.T @ qh)
            dv[b, :, g] += p.T @ doh
    return dq, dk, dv


def backward_magnitudes(q, k, v, do, causal=False, scale=None, window=(-1, -1)):
    """fp64 magnitudes (mq, mk, mv) of the sums behind backward()'s gradients.

    Each gradient element is a sum of terms; a sum whose terms carry relative
    errors u has an error of at most u times the sum of the terms' absolute
    values, which is what this returns, with the row term D_i = sum_c dO O
    counted by its own magnitude (an implementation forms D from its rounded O):
      mv = sum_i P_ij |dO_ic|,
      aS_ij = P_ij (|dP_ij - D_i| + sum_c |dO_ic O_ic|),
      mq = |scale| sum_j aS_ij |K_jc|,  mk = |scale| sum_i aS_ij |Q_ic|,
    group-summed over the query heads of a key/value head like the gradients."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv
    vis = mask_matrix(Nq, Nk, causal, window)
    has = vis.any(axis=1)
    mq = np.zeros_like(q)
    mk = np.zeros_like(k)
    mv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh, kh, vh, doh = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
            s = scale * (qh @ kh.T)
            s = np.where(vis, s, -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            p = e / np.where(has, e.sum(axis=1), 1.0)[:, None]
            o = p @ vh
            dp = doh @ vh.T
            dd = (doh * o).sum(axis=1)
            a_s = p * (np.abs(dp - dd[:, None]) + np.abs(doh * o).sum(axis=1)[:, None])
            mq[b, :, h] = abs(scale) * (a_s @ np.abs(kh))
            mk[b, :, g] += abs(scale) * (a_s.T @ np.abs(qh))
            mv[b, :, g] += p.T @ np.abs(doh)
    return mq, mk, mv


def backward_operand_sums(q, k, do, causal=False, scale=None, window=(-1, -1)):
    """fp64 sums (fq, fk, fv) of the factors that multiply P and dS in backward()'s
    products, over the (row, key) pairs that see each other:
      fv[j, c] = sum_i |dO_ic|,  fk[j, c] = |scale| sum_i |Q_ic|,  fq[i, c] = |scale| sum_j |K_jc|,
    group-summed over the query heads of a key/value head like the gradients.
    Rounding a probability or a dS value to a 16-bit type where it lies below the
    type's normal range has an absolute error of up to half the subnormal spacing
    rather than a relative one; these sums carry that error into each gradient
    element (q and k as [B, N, H, d], do like q)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    do = np.asarray(do, np.float64)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = Hq // Hkv
    vis = mask_matrix(Nq, Nk, causal, window).astype(np.float64)
    fq = np.zeros_like(q)
    fk = np.zeros_like(k)
    fv = np.zeros_like(k)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            fq[b, :, h] = abs(scale) * (vis @ np.abs(k[b, :, g]))
            fk[b, :, g] += abs(scale) * (vis.T @ np.abs(q[b, :, h]))
            fv[b, :, g] += vis.T @ np.abs(do[b, :, h])
    return fq, fk, fv
