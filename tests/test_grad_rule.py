"""CPU pins of the gradient tolerance: oracle.backward_magnitudes and
oracle.backward_operand_sums against closed forms, and the element-wise rule of
_compare.check_grad against mistakes planted in a copy of the oracle's gradient
arithmetic (on the CPU), against a plain float32 implementation of the kernels'
arithmetic, and on a subnormal fp16 probability worked by hand.

backward_magnitudes sets the scale of every dQ, dK, dV tolerance, so it is pinned
from both sides: exact values where the sums have a closed form (one visible key,
and a two-key case worked out by hand), and planted mistakes that any loosened
magnitude would let through must still fail by a wide margin.
"""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic


def rand(*shape, seed=[0]):
    seed[0] += 1
    return np.random.default_rng([77, seed[0]]).standard_normal(shape)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_magnitudes_with_one_visible_key(causal):
    """One key: P = 1 for it, so O_i = V_0 and dP_i0 = D_i = sum_c dO_ic V_0c; the
    term |dP - D| vanishes and aS_i0 = sum_c |dO_ic V_0c|. Hence
      mq[i, c] = |scale| (sum_c' |dO_ic' V_0c'|) |K_0c|,
      mk[0, c] = |scale| sum_{h in group, i} (sum_c' |dO_ic' V_0c'|) |Q_ic|,
      mv[0, c] = sum_{h in group, i} |dO_ic|,
    over the rows that see the key (causal with Nq = 3 > Nk = 1: only row 2)."""
    B, Nq, Nk, Hq, Hkv, d = 2, 3, 1, 4, 2, 5
    q, k, v, do = rand(B, Nq, Hq, d), rand(B, Nk, Hkv, d), rand(B, Nk, Hkv, d), rand(B, Nq, Hq, d)
    scale = -0.7
    mq, mk, mv = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=scale)
    group = Hq // Hkv
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Nq):
                if causal and 0 > i + Nk - Nq:
                    continue   # row i sees no key
                a = sum(abs(do[b, i, h, c] * v[b, 0, g, c]) for c in range(d))
                for c in range(d):
                    eq[b, i, h, c] = abs(scale) * a * abs(k[b, 0, g, c])
                    ek[b, 0, g, c] += abs(scale) * a * abs(q[b, i, h, c])
                    ev[b, 0, g, c] += abs(do[b, i, h, c])
    np.testing.assert_allclose(mq, eq, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(mk, ek, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(mv, ev, rtol=1e-13, atol=1e-300)


def test_two_keys_worked_by_hand():
    """One query, two keys, d = 1, scale 1: q = 1, k = (0, ln 3), v = (2, -2), dO = 1.
    Scores (0, ln 3) give P = (1/4, 3/4); O = 2/4 - 6/4 = -1; dP = dO v = (2, -2);
    D = dO O = -1; dP - D = (3, -1); dS = P (dP - D) = (3/4, -3/4).
    Gradients: dQ = dS . k = -3/4 ln 3, dK = dS q = (3/4, -3/4), dV = P dO = (1/4, 3/4).
    Magnitudes: aS = P (|dP - D| + |dO O|) = (1/4 * 4, 3/4 * 2) = (1, 3/2);
    mq = 1 * |0| + 3/2 * ln 3, mk = aS |q| = (1, 3/2), mv = P |dO| = (1/4, 3/4).
    (|dP| + |D| in place of |dP - D| would give aS = (1, 3); dropping |dO O| would
    give (3/4, 3/4); both differ here.)"""
    ln3 = math.log(3.0)
    q = np.array([1.0]).reshape(1, 1, 1, 1)
    k = np.array([0.0, ln3]).reshape(1, 2, 1, 1)
    v = np.array([2.0, -2.0]).reshape(1, 2, 1, 1)
    do = np.array([1.0]).reshape(1, 1, 1, 1)
    o, lse = oracle.attention(q, k, v, scale=1.0)
    np.testing.assert_allclose(o.ravel(), [-1.0], atol=1e-15)
    np.testing.assert_allclose(lse.ravel(), [math.log(4.0)], atol=1e-15)
    dq, dk, dv = oracle.backward(q, k, v, do, scale=1.0)
    np.testing.assert_allclose(dq.ravel(), [-0.75 * ln3], atol=1e-15)
    np.testing.assert_allclose(dk.ravel(), [0.75, -0.75], atol=1e-15)
    np.testing.assert_allclose(dv.ravel(), [0.25, 0.75], atol=1e-15)
    mq, mk, mv = oracle.backward_magnitudes(q, k, v, do, scale=1.0)
    np.testing.assert_allclose(mq.ravel(), [1.5 * ln3], atol=1e-15)
    np.testing.assert_allclose(mk.ravel(), [1.0, 1.5], atol=1e-15)
    np.testing.assert_allclose(mv.ravel(), [0.25, 0.75], atol=1e-15)


# ---------------------------------------------------------------- planted mistakes

def planted_backward(q, k, v, do, causal, scale, mistake):
    """The oracle's gradient arithmetic with one mistake planted (CPU only):
    'drop_D' forms dS = P * dP without the row term D; 'mask_shift' lets every causal
    row see one key past its diagonal; 'swap_dO' swaps the upstream gradients of
    query rows 3 and 4."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    vis = oracle.mask_matrix(Nq, Nk, causal)
    if mistake == "mask_shift":
        vis = oracle.mask_matrix(Nq, Nk, False, (-1, 1))
    if mistake == "swap_dO":
        do = do.copy()
        do[:, [3, 4]] = do[:, [4, 3]]
    has = vis.any(axis=1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            qh, kh, vh, doh = q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h]
            s = np.where(vis, scale * (qh @ kh.T), -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            p = e / np.where(has, e.sum(axis=1), 1.0)[:, None]
            dp = doh @ vh.T
            ds = p * dp if mistake == "drop_D" else p * (dp - (p * dp).sum(axis=1)[:, None])
            dq[b, :, h] = scale * (ds @ kh)
            dk[b, :, g] += scale * (ds.T @ qh)
            dv[b, :, g] += p.T @ doh
    return dq, dk, dv


def case(dtype, causal):
    """The GPU tests' head-dim shape (B 2, Nq 200, Nk 333, 6 query heads over 2 KV heads)
    at d = 64, as exact 16-bit values."""
    B, Nq, Nk, Hq, Hkv, d = 2, 200, 333, 6, 2, 64
    bits = [synthetic.normal_bits(4000, t, s, dtype)
            for t, s in ((0, (B, Nq, Hq, d)), (1, (B, Nk, Hkv, d)), (2, (B, Nk, Hkv, d)), (3, (B, Nq, Hq, d)))]
    return [oracle.widen(x, dtype) for x in bits] + [1.0 / math.sqrt(d)]


# the smallest ratio to u M a planted mistake must reach: five times the rule's bound
MARGIN = 5 * cmp.GRAD_BOUND


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mistake", ["drop_D", "mask_shift", "swap_dO"])
def test_rule_rejects_planted_mistakes(dtype, causal, mistake):
    if mistake == "mask_shift" and not causal:
        pytest.skip("no diagonal to shift without a mask")
    q, k, v, do, sc = case(dtype, causal)
    ref = oracle.backward(q, k, v, do, causal=causal, scale=sc)
    mag = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=sc)
    bad = planted_backward(q, k, v, do, causal, sc, mistake)
    # the mistake in exact arithmetic, then rounded to the output type like a kernel's result
    bad = [oracle.widen(synthetic.to_bits(g.astype(np.float32), dtype), dtype) for g in bad]
    worst = max(float(cmp.grad_ratios(g, r, m, dtype).max()) for g, r, m in zip(bad, ref, mag))
    assert worst >= MARGIN, f"{mistake}: worst ratio {worst:.3g} below {MARGIN}"
    with pytest.raises(AssertionError):
        for g, r, m, n in zip(bad, ref, mag, ("dq", "dk", "dv")):
            cmp.check_grad(g, r, m, dtype, n)
    # and the pages' rule (twice a plain float32 implementation's error) rejects it too
    base = cmp.emulate_backward(q, k, v, do, causal, sc, dtype)
    with pytest.raises(AssertionError):
        for g, r, e, n in zip(bad, ref, base, ("dq", "dk", "dv")):
            cmp.check_grad_vs_baseline(g, r, e, dtype, n)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_rule_accepts_float32_arithmetic(dtype, causal):
    """A plain float32 implementation of the kernels' arithmetic (P and dS rounded to
    the input type as product operands, D from the rounded O) stays within one u M
    per element, half the rule's bound."""
    q, k, v, do, sc = case(dtype, causal)
    ref = oracle.backward(q, k, v, do, causal=causal, scale=sc)
    mag = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=sc)
    emu = cmp.emulate_backward(q, k, v, do, causal, sc, dtype)
    for g, r, m, n in zip(emu, ref, mag, ("dq", "dk", "dv")):
        assert cmp.check_grad(g, r, m, dtype, n) <= 1.0


# ------------------------------------------------- the rounding below normal range

@pytest.mark.parametrize("causal", [False, True])
def test_operand_sums_with_one_visible_key(causal):
    """One key: every row that sees it multiplies its P (and dS) by dO (and Q, K) once:
      fv[0, c] = sum_{h in group, i} |dO_ic|,  fk[0, c] = |scale| sum_{h in group, i} |Q_ic|,
      fq[i, c] = |scale| |K_0c|,
    over the rows that see the key (causal with Nq = 3 > Nk = 1: only row 2)."""
    B, Nq, Nk, Hq, Hkv, d = 2, 3, 1, 4, 2, 5
    q, k, do = rand(B, Nq, Hq, d), rand(B, Nk, Hkv, d), rand(B, Nq, Hq, d)
    scale = -0.7
    fq, fk, fv = oracle.backward_operand_sums(q, k, do, causal=causal, scale=scale)
    group = Hq // Hkv
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(k)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Nq):
                if causal and i < Nq - 1:
                    continue   # only the last row sees the key
                for c in range(d):
                    eq[b, i, h, c] = abs(scale) * abs(k[b, 0, g, c])
                    ek[b, 0, g, c] += abs(scale) * abs(q[b, i, h, c])
                    ev[b, 0, g, c] += abs(do[b, i, h, c])
    np.testing.assert_allclose(fq, eq, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(fk, ek, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(fv, ev, rtol=1e-13, atol=1e-300)


def test_operand_sums_count_each_visible_pair_once():
    """Causal, Nq = Nk = 4, d = 1, every |Q| = |K| = |dO| = 1, scale 1: key j is
    seen by rows j..3 and row i sees keys 0..i, so fv = fk = (4, 3, 2, 1) and
    fq = (1, 2, 3, 4)."""
    one = np.ones((1, 4, 1, 1))
    fq, fk, fv = oracle.backward_operand_sums(one, -one, one, causal=True, scale=1.0)
    np.testing.assert_array_equal(fv[0, :, 0, 0], [4, 3, 2, 1])
    np.testing.assert_array_equal(fk[0, :, 0, 0], [4, 3, 2, 1])
    np.testing.assert_array_equal(fq[0, :, 0, 0], [1, 2, 3, 4])


def test_subnormal_probability_needs_the_absolute_term():
    """One query, two keys, d = 1, scale 1, fp16: q = 1, k = (0, s), v = (0, 1),
    dO = 3, with s chosen so that P_1 = 6.28e-6 lies between two fp16 subnormals
    (spacing 2^-24). dV_1 = 3 P_1 (itself subnormal); an implementation that rounds
    P_1 to fp16 as the product operand and the product to fp16 is off by about 1.2
    spacings, 0.4% of dV_1: beyond half an ulp of the result plus 2 u M with the
    relative roundoff u = 2^-11 alone, within 2 (u M + eta F)."""
    p1 = 105.4 * 2.0 ** -24
    s = math.log(p1 / (1.0 - p1))
    q = np.ones((1, 1, 1, 1))
    k = np.array([0.0, s]).reshape(1, 2, 1, 1)
    v = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    do = np.full((1, 1, 1, 1), 3.0)
    ref = oracle.backward(q, k, v, do, scale=1.0)
    mag = oracle.backward_magnitudes(q, k, v, do, scale=1.0)
    flo = oracle.backward_operand_sums(q, k, do, scale=1.0)
    np.testing.assert_allclose(ref[2][0, 1, 0, 0], 3.0 * p1, rtol=1e-12)
    np.testing.assert_allclose(flo[2][0, 1, 0, 0], 3.0, rtol=0)
    got = ref[2].copy()
    got[0, 1, 0, 0] = float(np.float16(float(np.float16(p1)) * 3.0))
    assert abs(got[0, 1, 0, 0] - 3.0 * p1) > 2.0 ** -24
    with pytest.raises(AssertionError):
        cmp.check_grad(got, ref[2], mag[2], "f16", "dv without the absolute term")
    assert cmp.check_grad(got, ref[2], mag[2], "f16", "dv", floor=flo[2]) <= 1.0
