"""Tolerance rules used by the GPU parity tests.

Output O (fp16/bf16) against the fp64 oracle:
  max over elements of  (|O_gpu - O_ref| - ulp(O_ref)/2)    <= 1e-2
  mean over elements of max(0, |O_gpu - O_ref| - ulp(O_ref)/2) <= 1e-3
The half-ulp allowance is the error of rounding the exact result to the output
type; without it no bf16 output could meet 1e-2 where |O| >= 4 (bf16 spacing
there is 2^-5), nor the mean bound where |O| is near 1 (a sequence of two keys:
the correctly rounded bf16 result alone is 9.1e-4 off on average). LSE (fp32):
|LSE_gpu - LSE_ref| <= 1e-3 where finite, and both -inf exactly where a row
sees no key.

Gradients dQ, dK, dV (fp16/bf16) against the fp64 oracle, element by element:
  |G_gpu - G_ref| - ulp(G_ref)/2 <= 2 (u M + eta F)
with u the unit roundoff of the input type (2^-8 bf16, 2^-11 fp16), M the
sum of the magnitudes of the terms the element adds up (oracle
backward_magnitudes), eta half the type's smallest subnormal spacing (2^-25
fp16, 2^-134 bf16) and F the sum of the magnitudes of the factors P and dS are
multiplied by (oracle backward_operand_sums; callers that pass none get F = 0).
An implementation that rounds P and dS to the input type as MFMA operands,
accumulates in fp32 and forms D from its rounded O has an error of at most about
u M + eta F: the rounding is relative (u) in the normal range and absolute (eta)
below it, where a probability of a key that a single row barely sees can land
(fp16 P near 6e-6: half an ulp is 0.5% of it). A float32 emulation of that
arithmetic reaches 0.84 u M on the test shapes, and a dropped D term, a causal
mask one key off or two swapped dO rows exceed the bound 3x to 10^5x.

Secondary rule (the upstream test criterion, "flash-attention-v100" README,
Tests: the output and the gradients have at most twice the error of a baseline
implementation): max error <= 2 * max error of a float32 emulation (fp32 scores
and softmax, P rounded to the input type, fp32 P V, O rounded; for the
gradients the same arithmetic as emulate_backward) plus one output ulp of slack
for the rounding of the result itself; for gradients with at least 4096
non-zero reference elements (below that the two maxima are draws of a few
roundings and the element-wise rule alone applies).
"""
from __future__ import annotations

import math

import numpy as np

MAX_TOL = 1e-2
MEAN_TOL = 1e-3
LSE_TOL = 1e-3
MANT = {"f16": 10, "bf16": 7}
MIN_EXP = {"f16": -14, "bf16": -126}


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit type at |x| (normal range; subnormal spacing below it)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, MIN_EXP[dtype])
    return np.exp2(e - MANT[dtype])


def check_o(o_gpu, o_ref, dtype, what=""):
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    excess = err - 0.5 * ulp(o_ref, dtype)
    worst = float(excess.max()) if err.size else 0.0
    mean = float(np.maximum(excess, 0.0).mean()) if err.size else 0.0
    stats = dict(max_err=float(err.max()) if err.size else 0.0, max_excess=worst,
                 mean_err=float(err.mean()) if err.size else 0.0, mean_excess=mean)
    assert worst <= MAX_TOL, f"{what}: max |dO| - ulp/2 = {worst:.3g} > {MAX_TOL} {stats}"
    assert mean <= MEAN_TOL, f"{what}: mean (|dO| - ulp/2)+ = {mean:.3g} > {MEAN_TOL} {stats}"
    return stats


UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
SUBNORMAL_HALF = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}
GRAD_BOUND = 2.0


def grad_bound(mag, dtype, floor=None):
    """u M + eta F per element (F = 0 without `floor`)."""
    b = UNIT_ROUNDOFF[dtype] * np.asarray(mag, np.float64)
    if floor is not None:
        b = b + SUBNORMAL_HALF[dtype] * np.asarray(floor, np.float64)
    return b


def grad_ratios(g_gpu, g_ref, mag, dtype, floor=None):
    """Per element: (|G - G_ref| - ulp(G_ref)/2) / (u M + eta F), 0 where within half an ulp."""
    g_gpu = np.asarray(g_gpu, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    excess = np.abs(g_gpu - g_ref) - 0.5 * ulp(g_ref, dtype)
    bound = grad_bound(mag, dtype, floor)
    return np.where(excess > 0, excess / np.maximum(bound, 1e-300), 0.0)


def check_grad(g_gpu, g_ref, mag, dtype, what="", floor=None):
    """Element-wise rounding-error bound on a gradient (rule above)."""
    g_gpu = np.asarray(g_gpu, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    assert g_gpu.shape == g_ref.shape, (g_gpu.shape, g_ref.shape)
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite gradient"
    bound = grad_bound(mag, dtype, floor)
    ratio = grad_ratios(g_gpu, g_ref, mag, dtype, floor)
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > GRAD_BOUND:
        i = np.unravel_index(int(ratio.argmax()), ratio.shape)
        raise AssertionError(f"{what}: |dG| = {abs(g_gpu[i] - g_ref[i]):.3g} at {i} exceeds {GRAD_BOUND} (u M + eta F) "
                             f"(u M + eta F = {bound[i]:.3g}, ref {g_ref[i]:.3g}, gpu {g_gpu[i]:.3g}); "
                             f"ratio {worst:.3g}")
    return worst


def check_lse(lse_gpu, lse_ref, what=""):
    lse_gpu = np.asarray(lse_gpu, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    assert lse_gpu.shape == lse_ref.shape
    ninf_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse_gpu), ninf_ref, err_msg=f"{what}: -inf rows differ")
    fin = ~ninf_ref
    assert np.all(np.isfinite(lse_gpu[fin])), f"{what}: non-finite LSE"
    d = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert d <= LSE_TOL, f"{what}: max |dLSE| = {d:.3g} > {LSE_TOL}"
    return d


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32)


def emulate_rows(q, k, v, rows, h, causal, scale, dtype, nq):
    """Float32 baseline for query rows `rows` of one (batch, head): q [Nq,d], k/v [Nk,d] float64."""
    q32 = np.asarray(q[rows], np.float32)
    k32 = np.asarray(k, np.float32)
    v32 = np.asarray(v, np.float32)
    s = (q32 @ k32.T) * np.float32(scale)
    nk = k.shape[0]
    if causal:
        lim = np.asarray(rows)[:, None] + (nk - nq)
        s = np.where(np.arange(nk)[None, :] <= lim, s, -np.inf).astype(np.float32)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0).astype(np.float32)
    p = np.exp(s - m).astype(np.float32)
    l = p.sum(axis=1, keepdims=True)
    o = (_round_to(p, dtype) @ v32) / np.where(l > 0, l, 1)
    return _round_to(o, dtype).astype(np.float64)


def _visible(nq, nk, causal, window):
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    diag = i + nk - nq
    m = np.ones((nq, nk), bool)
    if causal:
        m &= j <= diag
    if window[0] >= 0:
        m &= j >= diag - window[0]
    if window[1] >= 0:
        m &= j <= diag + window[1]
    return m


def emulate_backward(q, k, v, do, causal, scale, dtype, window=(-1, -1)):
    """Float32 baseline of the gradients: q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d], do like q
    (exact 16-bit values as float64). A plain low-precision implementation of the
    same arithmetic: fp32 scores and softmax, O rounded to the input type and
    D = rowsum(dO * O) from it, P and dS rounded to the input type as product
    operands, fp32 products and sums, gradients rounded to the input type; a KV
    head sums its query heads' terms in fp32 before rounding."""
    q32, k32, v32, do32 = (np.asarray(x, np.float32) for x in (q, k, v, do))
    B, Nq, Hq, d = q32.shape
    Nk, Hkv = k32.shape[1], k32.shape[2]
    group = Hq // Hkv
    vis = _visible(Nq, Nk, causal, window)
    has = vis.any(axis=1)
    sc = np.float32(scale)
    dq = np.zeros((B, Nq, Hq, d), np.float32)
    dk = np.zeros((B, Nk, Hkv, d), np.float32)
    dv = np.zeros((B, Nk, Hkv, d), np.float32)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh, kh, vh, doh = q32[b, :, h], k32[b, :, g], v32[b, :, g], do32[b, :, h]
            s = np.where(vis, (qh @ kh.T) * sc, -np.inf).astype(np.float32)
            m = np.where(has, s.max(axis=1), 0).astype(np.float32)
            e = np.where(vis, np.exp(s - m[:, None]), 0).astype(np.float32)
            p = (e / np.where(has, e.sum(axis=1), 1)[:, None]).astype(np.float32)
            o = _round_to(_round_to(p, dtype) @ vh, dtype)
            dp = doh @ vh.T
            dd = (doh * o).sum(axis=1, dtype=np.float32)
            ds = (p * (dp - dd[:, None])).astype(np.float32)
            dq[b, :, h] = sc * (_round_to(ds, dtype) @ kh)
            dk[b, :, g] += sc * (_round_to(ds, dtype).T @ qh)
            dv[b, :, g] += _round_to(p, dtype).T @ doh
    return tuple(_round_to(x, dtype).astype(np.float64) for x in (dq, dk, dv))


# the comparison of two maxima needs enough elements to be more than a draw of a
# few roundings; smaller gradients are held to the element-wise rule alone
BASELINE_MIN_ELEMS = 4096


def check_grad_vs_baseline(g_gpu, g_ref, g_base, dtype, what=""):
    """The pages' test criterion on a gradient tensor: its maximum error against the
    fp64 oracle is at most twice that of the plain float32 baseline, plus one output
    ulp of the largest reference value for the rounding of the gradient itself.
    Applied where the reference has at least BASELINE_MIN_ELEMS non-zero elements:
    in a windowed 19 x 2 case with 512 of them the largest dQ error of a correct
    kernel was 2.5 times the baseline's, and 1/20 of its element-wise bound, since
    each element there is the rounding of two large cancelling terms."""
    g_gpu, g_ref, g_base = (np.asarray(x, np.float64) for x in (g_gpu, g_ref, g_base))
    e_gpu = float(np.abs(g_gpu - g_ref).max()) if g_ref.size else 0.0
    e_base = float(np.abs(g_base - g_ref).max()) if g_ref.size else 0.0
    if np.count_nonzero(g_ref) < BASELINE_MIN_ELEMS:
        return e_gpu, e_base
    slack = float(ulp(np.abs(g_ref).max(), dtype)) if g_ref.size else 0.0
    assert e_gpu <= 2 * e_base + slack, f"{what}: max error {e_gpu:.3g} > 2 x baseline {e_base:.3g} + {slack:.3g}"
    return e_gpu, e_base


def sample_rows(n: int, rng: np.random.Generator, extra: int = 64):
    base = {0, 1, 31, 32, 127, 128, n // 2, n - 2, n - 1}
    base |= set(int(x) for x in rng.choice(n, size=min(extra, n), replace=False))
    return sorted(r for r in base if 0 <= r < n)


def fmt(stats: dict) -> str:
    return " ".join(f"{k}={v:.3g}" for k, v in stats.items())


def nan_to_str(x):  # pragma: no cover - message helper
    return "nan" if isinstance(x, float) and math.isnan(x) else str(x)
