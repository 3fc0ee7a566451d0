"""Pins for the fp64 oracle: each test ties it to something other than itself.

Sources: the pages' worked examples (golden fixtures), closed forms,
special cases, invariants, and an independent pure-Python brute force.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def onehot_v(B, Nk, Hkv, d):
    """V[b, j, g, :] = e_j, so O[i, :Nk] is the probability row of query i."""
    assert d >= Nk
    v = np.zeros((B, Nk, Hkv, d))
    for j in range(Nk):
        v[:, j, :, j] = 1.0
    return v


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("nq,nk,fixture", [(2, 5, "causal_mask_q2_k5.txt"), (5, 2, "causal_mask_q5_k2.txt")])
def test_causal_mask_matches_pages_examples(golden, nq, nk, fixture):
    mask = golden(fixture)
    assert mask.shape == (nq, nk)
    q = rand(1, nq, 1, 8)
    k = rand(1, nk, 1, 8)
    v = onehot_v(1, nk, 1, 8)
    o, lse = oracle.attention(q, k, v, causal=True)
    probs = o[0, :, 0, :nk]
    np.testing.assert_array_equal((probs > 0).astype(int), mask)
    # rows with no visible key: all-zero output and LSE = -inf
    for i in range(nq):
        if mask[i].sum() == 0:
            assert np.all(o[0, i, 0] == 0.0)
            assert lse[0, 0, i] == -math.inf
        else:
            assert np.isfinite(lse[0, 0, i])
            assert abs(probs[i].sum() - 1.0) < 1e-12


def test_causal_mask_is_not_top_left_aligned(golden):
    old = golden("causal_mask_q2_k5_v20.txt")
    v = onehot_v(1, 5, 1, 8)
    o, _ = oracle.attention(rand(1, 2, 1, 8), rand(1, 5, 1, 8), v, causal=True)
    assert not np.array_equal((o[0, :, 0, :5] > 0).astype(int), old)


def test_gqa_head_map_matches_pages_example(golden):
    table = golden("gqa_heads_6_over_2.txt")
    Hq, Hkv, d, Nk = 6, 2, 4, 7
    q = rand(2, 3, Hq, d)
    k = rand(2, Nk, Hkv, d)
    v = np.zeros((2, Nk, Hkv, d))
    v[:, :, 0, :] = 1.0
    v[:, :, 1, :] = 2.0          # each KV head has a constant value: O names the head read
    o, _ = oracle.attention(q, k, v)
    for h, g in table:
        np.testing.assert_allclose(o[:, :, h, :], g + 1.0, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    Hq, Hkv = 6, 2
    q, k, v = rand(2, 5, Hq, 8), rand(2, 9, Hkv, 8), rand(2, 9, Hkv, 8)
    o1, l1 = oracle.attention(q, k, v, causal=True)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    o2, l2 = oracle.attention(q, kr, vr, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    B, N, H, d = 2, 11, 3, 5
    q = np.zeros((B, N, H, d))
    k, v = rand(B, N, H, d), rand(B, N, H, d)
    o, lse = oracle.attention(q, k, v, causal=causal)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(o[:, i], v[:, :n].mean(axis=1), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14)


def test_single_key_gives_that_value_row():
    q, k, v = rand(2, 4, 4, 16), rand(2, 1, 2, 16), rand(2, 1, 2, 16)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, scale=scale)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(o[:, :, h], np.broadcast_to(v[:, 0:1, g], o[:, :, h].shape), atol=1e-15)
        want = scale * np.einsum("bic,bc->bi", q[:, :, h], k[:, 0, g])
        np.testing.assert_allclose(lse[:, h], want, rtol=1e-14, atol=1e-14)


def test_causal_row_zero_is_first_value_row():
    q, k, v = rand(1, 6, 2, 8), rand(1, 6, 2, 8), rand(1, 6, 2, 8)
    o, lse = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], (q[0, 0] * k[0, 0]).sum(-1) / math.sqrt(8), rtol=1e-14)


@pytest.mark.parametrize("x", [-3.0, -0.5, 0.0, 0.75, 4.0])
def test_two_keys_is_a_logistic(x):
    # d = 1, q = 1, keys 0 and x/scale, values 0 and 1: O = e^x / (1 + e^x)
    scale = 0.125
    q = np.ones((1, 1, 1, 1))
    k = np.array([0.0, x / scale]).reshape(1, 2, 1, 1)
    v = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    o, lse = oracle.attention(q, k, v, scale=scale)
    assert abs(o[0, 0, 0, 0] - 1.0 / (1.0 + math.exp(-x))) < 1e-15
    assert abs(lse[0, 0, 0] - math.log1p(math.exp(x))) < 1e-14


def test_default_scale_is_inverse_sqrt_head_dim():
    q, k, v = rand(1, 3, 1, 16), rand(1, 5, 1, 16), rand(1, 5, 1, 16)
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q * 0.25, k, v, scale=1.0)   # 1/sqrt(16) = 0.25, exact
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)


# ---------------------------------------------------------------- invariants

def test_key_permutation_invariance_non_causal():
    q, k, v = rand(2, 7, 2, 8), rand(2, 13, 2, 8), rand(2, 13, 2, 8)
    perm = RNG.permutation(13)
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_causal_row_equals_prefix_attention():
    q, k, v = rand(1, 9, 2, 8), rand(1, 9, 2, 8), rand(1, 9, 2, 8)
    o, lse = oracle.attention(q, k, v, causal=True)
    for i in range(9):
        oi, li = oracle.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1])
        np.testing.assert_allclose(o[:, i], oi[:, 0], atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], li[:, :, 0], atol=1e-14)


def test_linearity_in_values():
    q, k = rand(1, 5, 2, 8), rand(1, 9, 2, 8)
    v1, v2 = rand(1, 9, 2, 8), rand(1, 9, 2, 8)
    a, b = 1.75, -0.5
    o1, _ = oracle.attention(q, k, v1, causal=True)
    o2, _ = oracle.attention(q, k, v2, causal=True)
    o3, _ = oracle.attention(q, k, a * v1 + b * v2, causal=True)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-13)


def test_output_is_a_convex_combination():
    q, k, v = 3 * rand(1, 8, 2, 8), 3 * rand(1, 12, 2, 8), rand(1, 12, 2, 8)
    o, _ = oracle.attention(q, k, v)
    assert np.all(o <= v.max(axis=1, keepdims=True) + 1e-14)
    assert np.all(o >= v.min(axis=1, keepdims=True) - 1e-14)


@pytest.mark.parametrize("ranges", [[(0, 37)], [(0, 5), (5, 6), (6, 20), (20, 21), (21, 30), (30, 33), (33, 37)],
                                    [(16 * s, min(37, 16 * s + 16)) for s in range(3)]])
def test_split_combine_equals_unsplit(ranges):
    q, k, v = rand(2, 3, 4, 8), rand(2, 37, 2, 8), rand(2, 37, 2, 8)
    o_ref, l_ref = oracle.attention(q, k, v)
    parts = [oracle.attention(q, k, v, key_range=r) for r in ranges]
    o, lse = oracle.combine_splits([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, atol=1e-13)


def test_sixteen_even_splits_with_empty_chunk_rows():
    # causal, Nq = 8 over 64 keys in 16 chunks of 4: early chunks are empty for no
    # row, late chunks are empty for early rows (LSE_s = -inf must weigh nothing)
    q, k, v = rand(1, 8, 2, 8), rand(1, 64, 2, 8), rand(1, 64, 2, 8)
    o_ref, l_ref = oracle.attention(q, k, v, causal=True)
    parts = [oracle.attention(q, k, v, causal=True, key_range=(4 * s, 4 * s + 4)) for s in range(16)]
    assert any(np.isneginf(p[1]).any() for p in parts)
    o, lse = oracle.combine_splits([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, atol=1e-13)


def test_combine_of_all_empty_chunks_is_zero():
    o = np.ones((3, 1, 1, 1, 4))
    lse = np.full((3, 1, 1, 1), -np.inf)
    oc, lc = oracle.combine_splits(o, lse)
    assert np.all(oc == 0) and np.all(np.isneginf(lc))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,window", [
    (1, 4, 4, 1, 1, 3, False, (-1, -1)),
    (2, 5, 7, 6, 2, 4, True, (-1, -1)),
    (1, 7, 3, 2, 1, 8, True, (-1, -1)),
    (1, 9, 9, 4, 4, 5, True, (-1, -1)),
    (2, 6, 9, 3, 1, 2, False, (2, 1)),
    (1, 6, 6, 2, 2, 3, True, (1, -1)),
])
def test_matches_pure_python_brute_force(B, Nq, Nk, Hq, Hkv, d, causal, window):
    q, k, v = rand(B, Nq, Hq, d), rand(B, Nk, Hkv, d), rand(B, Nk, Hkv, d)
    o1, l1 = oracle.attention(q, k, v, causal=causal, window=window)
    o2, l2, probs = oracle.brute_force(q, k, v, causal=causal, window=window, return_probs=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    rows = probs.sum(-1)
    has = np.isfinite(l2)
    np.testing.assert_allclose(rows[has], 1.0, atol=1e-12)      # rows of P sum to 1
    assert np.all(rows[~has] == 0)


def test_window_zero_zero_selects_the_diagonal_key():
    q, k, v = rand(1, 5, 1, 4), rand(1, 8, 1, 4), rand(1, 8, 1, 4)
    o, _ = oracle.attention(q, k, v, window=(0, 0))
    for i in range(5):
        np.testing.assert_allclose(o[0, i, 0], v[0, i + 3, 0], atol=1e-15)


def test_window_open_left_right_zero_equals_causal():
    # the causal mask is the band with no left limit and right edge 0
    q, k, v = rand(2, 9, 4, 6), rand(2, 13, 2, 6), rand(2, 13, 2, 6)
    o1, l1 = oracle.attention(q, k, v, window=(-1, 0))
    o2, l2 = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_window_wider_than_the_keys_changes_nothing():
    q, k, v = rand(1, 6, 2, 4), rand(1, 10, 2, 4), rand(1, 10, 2, 4)
    o1, l1 = oracle.attention(q, k, v, window=(50, 50))
    o2, l2 = oracle.attention(q, k, v)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)


@pytest.mark.parametrize("window", [(2, 1), (0, 3), (4, 0), (1, 1)])
def test_window_row_equals_plain_attention_over_its_key_slice(window):
    # each row of a band is plain (unmasked) attention over the slice of keys
    # [i + Nk - Nq - left, i + Nk - Nq + right], cut out in Python
    Nq, Nk = 6, 11
    q, k, v = rand(1, Nq, 2, 5), rand(1, Nk, 1, 5), rand(1, Nk, 1, 5)
    o, lse = oracle.attention(q, k, v, window=window)
    for i in range(Nq):
        lo = max(0, i + Nk - Nq - window[0])
        hi = min(Nk, i + Nk - Nq + window[1] + 1)
        ob, lb = oracle.attention(q[:, i:i + 1], k[:, lo:hi], v[:, lo:hi])
        np.testing.assert_allclose(o[:, i:i + 1], ob, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i:i + 1], lb, atol=1e-14)


def test_seqlens_k_equals_truncated_cache():
    q, k, v = rand(3, 2, 4, 8), rand(3, 20, 2, 8), rand(3, 20, 2, 8)
    lens = np.array([20, 7, 1], np.int32)
    o, lse = oracle.attention(q, k, v, causal=True, seqlens_k=lens)
    for b, n in enumerate(lens):
        ob, lb = oracle.attention(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], causal=True)
        np.testing.assert_allclose(o[b:b + 1], ob, atol=1e-14)
        np.testing.assert_allclose(lse[b:b + 1], lb, atol=1e-14)


# ---------------------------------------------------------------- storage formats

def test_widen_known_bit_patterns():
    f16 = np.array([0x3C00, 0x7BFF, 0x0001, 0x8000, 0xC500, 0x3555], np.uint16)
    np.testing.assert_array_equal(oracle.widen(f16, "f16"),
                                  [1.0, 65504.0, 2.0 ** -24, -0.0, -5.0, 0.333251953125])
    bf = np.array([0x3F80, 0xC0A0, 0x0001, 0x7F7F, 0x3EAB], np.uint16)
    np.testing.assert_array_equal(oracle.widen(bf, "bf16"),
                                  [1.0, -5.0, 2.0 ** -133, 3.3895313892515355e38, 0.333984375])


def test_rounding_helpers_are_nearest_even():
    # 1 + 2^-8 is a tie between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    np.testing.assert_array_equal(oracle.widen(synthetic.f32_to_bf16_bits(x), "bf16"),
                                  [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7])
    y = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11], np.float32)
    np.testing.assert_array_equal(oracle.widen(synthetic.f32_to_f16_bits(y), "f16"),
                                  [1.0, 1.0 + 2.0 ** -9])


def test_workload_inputs_are_seeded_and_sliceable():
    w = synthetic.WORKLOADS["tiny_f16_128"]
    q1, k1, v1 = w.inputs()
    q2, _, _ = w.inputs()
    np.testing.assert_array_equal(q1, q2)
    gq = synthetic.WORKLOADS["gqa_bf16_2048_d64"]
    qa, ka, _ = gq.inputs(batches=[3])
    assert qa.shape == (1, 2048, 32, 64) and ka.shape == (1, 2048, 8, 64)
    s = synthetic.WORKLOADS["long_bf16_8192_sharp_full"]
    assert s.qk_mult == 2.0 and s.dtype == "bf16"


def test_flop_convention_matches_pages_table():
    # The page-1 table divides 2*B*H*N^2*d by the time: 5.32 ms -> 25.84 TFLOP/s
    w = synthetic.WORKLOADS["headline_f16_1024"]
    assert abs(w.flops() / 2 / 5.32e-3 / 1e12 - 25.84) < 0.02
    assert w.pairs() == 1024 * 1024
    c = synthetic.WORKLOADS["long_f16_2048_causal"]
    assert c.pairs() == 2048 * 2049 // 2



# ---------------------------------------------------------------- backward

def test_mask_matrix_equals_visible():
    for Nq, Nk, causal, window in [(5, 5, True, (-1, -1)), (4, 9, False, (2, 1)), (9, 4, True, (1, -1)),
                                   (6, 6, False, (0, 0)), (3, 7, False, (-1, 2))]:
        m = oracle.mask_matrix(Nq, Nk, causal, window)
        for i in range(Nq):
            for j in range(Nk):
                assert m[i, j] == oracle.visible(i, j, Nq, Nk, causal, window)


def _loss(q, k, v, do, **kw):
    o, _ = oracle.attention(q, k, v, **kw)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (1, 1))])
def test_backward_matches_central_differences(causal, window):
    # the gradient of L = sum(dO * O) by finite differences of the forward oracle,
    # element by element: independent of the gradient formula
    B, Nq, Nk, Hq, Hkv, d = 1, 3, 5, 2, 1, 3
    q, k, v, do = rand(B, Nq, Hq, d), rand(B, Nk, Hkv, d), rand(B, Nk, Hkv, d), rand(B, Nq, Hq, d)
    dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, window=window)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, causal=causal, window=window)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, causal=causal, window=window)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8)


def test_backward_matches_torch_autograd_with_gqa():
    # torch autograd of a plainly written fp64 forward, with K/V heads repeated per group
    import torch
    B, Nq, Nk, Hq, Hkv, d = 2, 17, 23, 6, 2, 8
    q, k, v, do = rand(B, Nq, Hq, d), rand(B, Nk, Hkv, d), rand(B, Nk, Hkv, d), rand(B, Nq, Hq, d)
    scale = 0.37
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Hq // Hkv, dim=2)
    vv = tv.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", tq, kk) * scale
    mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("bhij,bjhc->bihc", torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv = oracle.backward(q, k, v, do, causal=True, scale=scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_rows_without_keys_have_zero_gradient():
    q, k, v, do = rand(1, 6, 2, 4), rand(1, 3, 2, 4), rand(1, 3, 2, 4), rand(1, 6, 2, 4)
    dq, dk, dv = oracle.backward(q, k, v, do, causal=True)
    # causal with Nq = 6 > Nk = 3: rows 0..2 see no key
    assert np.all(dq[0, :3] == 0) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))


def test_backward_magnitudes_bound_the_gradients():
    # triangle inequality: every gradient element is at most the sum of the magnitudes
    # of its terms, for masks, GQA and a negative scale alike
    for causal, window, scale in [(False, (-1, -1), None), (True, (-1, -1), 0.3), (False, (2, 0), -0.5)]:
        q, k, v, do = rand(2, 7, 4, 5), rand(2, 9, 2, 5), rand(2, 9, 2, 5), rand(2, 7, 4, 5)
        grads = oracle.backward(q, k, v, do, causal=causal, scale=scale, window=window)
        mags = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=scale, window=window)
        for g, m in zip(grads, mags):
            assert np.all(m >= 0)
            assert np.all(np.abs(g) <= m * (1 + 1e-12) + 1e-15)


def test_backward_magnitudes_equal_dv_for_nonnegative_do():
    # P >= 0, so with dO >= 0 every term of dV = P^T dO is non-negative: the magnitude is dV
    q, k, v, do = rand(1, 6, 4, 3), rand(1, 8, 2, 3), rand(1, 8, 2, 3), np.abs(rand(1, 6, 4, 3))
    _, _, dv = oracle.backward(q, k, v, do, causal=True)
    _, _, mv = oracle.backward_magnitudes(q, k, v, do, causal=True)
    np.testing.assert_allclose(mv, dv, rtol=1e-13, atol=1e-15)


def test_backward_magnitudes_are_homogeneous_in_do():
    # every term is linear in dO (D too), so all magnitudes scale with |c|
    q, k, v, do = rand(1, 5, 2, 4), rand(1, 6, 1, 4), rand(1, 6, 1, 4), rand(1, 5, 2, 4)
    a = oracle.backward_magnitudes(q, k, v, do, causal=True)
    b = oracle.backward_magnitudes(q, k, v, -3.0 * do, causal=True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, 3.0 * x, rtol=1e-12)
