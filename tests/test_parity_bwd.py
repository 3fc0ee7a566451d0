"""GPU parity of fa_bwd (dQ, dK, dV) against the fp64 oracle, through the C ABI.

Whole tensors at small sizes (several tiles, ragged tails, every head dim,
both dtypes, GQA groups, Nq != Nk, fully masked rows) with O and LSE from
fa_fwd, as a training step produces them, and with O and LSE from the oracle,
which checks the backward kernels on their own. At the pages' fwd+bwd benchmark
shape (B 4, N 4096, 16 heads of 128) the whole problem runs on the GPU in the
configuration the benchmark times, and whole heads of the first and last batch
element are checked. Criteria: an element-wise rounding-error bound (the
gradient rule of _compare), the pages' test criterion (max error at most twice
that of a plain float32 implementation, "flash-attention-v100" README, Tests),
and bit-identical results over repeated calls.
"""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention, attention_backward, attention_func  # noqa: E402

HEAD_DIMS = (32, 64, 96, 128, 192, 256)


def inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype):
    qb = synthetic.normal_bits(wid, synthetic.Q_ID, (B, Nq, Hq, d), dtype)
    kb = synthetic.normal_bits(wid, synthetic.K_ID, (B, Nk, Hkv, d), dtype)
    vb = synthetic.normal_bits(wid, synthetic.V_ID, (B, Nk, Hkv, d), dtype)
    dob = synthetic.normal_bits(wid, synthetic.DO_ID, (B, Nq, Hq, d), dtype)
    return qb, kb, vb, dob


def run_full(wid, B, Nq, Nk, Hq, Hkv, d, dtype, causal, scale=None, fwd="gpu", window=(-1, -1)):
    qb, kb, vb, dob = inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    what = (f"wid={wid} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal} fwd={fwd} "
            f"window={window}")
    print(f"[bwd] {what}", flush=True)
    q, k, v, do = (oracle.widen(x, dtype) for x in (qb, kb, vb, dob))
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (qb, kb, vb, dob))
    if fwd == "gpu":
        o, lse = attention(qd, kd, vd, causal=causal, scale=scale, window=window)
    else:
        import torch
        o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, scale=scale, window=window)
        o = to_dev(synthetic.to_bits(o_ref.astype(np.float32), dtype), dtype)
        lse = torch.from_numpy(lse_ref.astype(np.float32)).to(qd.device)
    dq, dk, dv = attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, window=window)
    ref = oracle.backward(q, k, v, do, causal=causal, scale=scale, window=window)
    mag = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=scale, window=window)
    flo = oracle.backward_operand_sums(q, k, do, causal=causal, scale=scale, window=window)
    got = [to_np(g) for g in (dq, dk, dv)]
    worst = [cmp.check_grad(g, r, m, dtype, f"{what} {n}", floor=f)
             for g, r, m, f, n in zip(got, ref, mag, flo, ("dq", "dk", "dv"))]
    # the pages' criterion: at most twice the error of a plain float32 implementation
    base = cmp.emulate_backward(q, k, v, do, causal, scale, dtype, window=window)
    errs = [cmp.check_grad_vs_baseline(g, r, e, dtype, f"{what} {n} vs float32 baseline")
            for g, r, e, n in zip(got, ref, base, ("dq", "dk", "dv"))]
    print(f"[bwd] ratio to u*M: dq {worst[0]:.3g} dk {worst[1]:.3g} dv {worst[2]:.3g}; max error / baseline's: "
          + " ".join(f"{a:.3g}/{b:.3g}" for a, b in errs), flush=True)
    return dq, dk, dv


EDGE = [
    (1, 9, 9, 12, 12, 64, "f16", False),      # GPT-2 sized example: seq 9, 12 heads, d 64
    (1, 9, 9, 12, 12, 64, "bf16", True),
    (2, 127, 129, 4, 2, 128, "bf16", True),
    (2, 129, 127, 4, 1, 128, "f16", True),    # Nq > Nk: first rows see no key
    (1, 300, 37, 2, 2, 64, "bf16", True),     # most rows fully masked
    (1, 37, 300, 2, 2, 64, "f16", True),
    (1, 1, 1, 1, 1, 32, "f16", False),
    (1, 1, 513, 2, 1, 128, "bf16", False),
    (1, 513, 1, 2, 1, 128, "bf16", False),
    (1, 256, 1000, 8, 8, 128, "f16", False),
    (3, 250, 250, 6, 6, 96, "bf16", False),
    (1, 160, 160, 8, 1, 64, "bf16", True),    # one KV head for 8 query heads
    (1, 3, 20001, 2, 1, 128, "bf16", False),  # a few rows over 20001 keys (157 key blocks)
    (1, 20001, 5, 2, 2, 128, "f16", True),    # 20001 rows over 5 keys: almost all rows see them all
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes(case):
    run_full(500 + EDGE.index(case), *case)


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims(d, dtype, causal):
    wid = 600 + HEAD_DIMS.index(d) * 4 + (dtype == "bf16") * 2 + int(causal)
    run_full(wid, 2, 200, 333, 6, 2, d, dtype, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_grouped_heads_order(causal, d):
    """32 (batch, head) pairs with 4 query heads per KV head: the work orders keep
    a KV group's query heads on one XCD (a permutation used only when the pair
    count is a multiple of 8 groups), in the dQ pass as in the forward."""
    run_full(97, 2, 300, 300, 16, 4, d, "bf16", causal)


@pytest.mark.parametrize("causal", [False, True])
def test_oracle_forward_inputs(causal):
    """O and LSE from the oracle: the backward kernels checked on their own."""
    run_full(650 + int(causal), 2, 257, 300, 4, 2, 128, "bf16", causal, fwd="oracle")
    run_full(652 + int(causal), 1, 300, 257, 4, 4, 64, "f16", causal, fwd="oracle")


def test_scale_is_used_as_passed():
    run_full(660, 1, 130, 130, 2, 2, 64, "f16", False, scale=0.37)
    run_full(661, 1, 130, 130, 2, 2, 64, "bf16", True, scale=-0.2)
    run_full(662, 1, 130, 130, 2, 2, 64, "bf16", True, scale=0.0)


def test_deterministic():
    """No atomics: repeated calls give bit-identical gradients."""
    import torch
    qb, kb, vb, dob = inputs(670, 2, 384, 384, 8, 2, 128, "bf16")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (qb, kb, vb, dob))
    o, lse = attention(qd, kd, vd, causal=True)
    first = attention_backward(qd, kd, vd, o, lse, dod, causal=True)
    for _ in range(3):
        again = attention_backward(qd, kd, vd, o, lse, dod, causal=True)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_autograd_function():
    """attention_func inside torch autograd gives the same gradients as the direct calls."""
    import torch
    qb, kb, vb, dob = inputs(680, 1, 200, 200, 4, 2, 64, "bf16")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (qb, kb, vb, dob))
    leaves = [t.clone().requires_grad_(True) for t in (qd, kd, vd)]
    out = attention_func(*leaves, causal=True)
    out.backward(dod)
    o, lse = attention(qd, kd, vd, causal=True)
    direct = attention_backward(qd, kd, vd, o, lse, dod, causal=True)
    assert torch.equal(out.view(torch.int16), o.view(torch.int16))
    for leaf, g in zip(leaves, direct):
        assert torch.equal(leaf.grad.view(torch.int16), g.view(torch.int16))


WINDOWS = [(0, 0), (16, 0), (100, 100), (-1, 50), (300, -1), (0, -1), (63, 64), (1000, 1000), (-1, 0)]


@pytest.mark.parametrize("window", WINDOWS, ids=lambda w: f"{w[0]}_{w[1]}")
def test_window(window):
    # several key and query tiles on both sides of the band, ragged tails
    run_full(700 + WINDOWS.index(window), 2, 333, 333, 4, 2, 128, "bf16", False, window=window)


@pytest.mark.parametrize("case", [(200, 450, False), (450, 200, False), (300, 300, True)],
                         ids=lambda c: "x".join(map(str, c)))
def test_window_alignment_and_causal(case):
    # bottom-right alignment with Nq != Nk both ways (rows or keys outside every band),
    # and causal fixing the right edge of a (left, right) window at 0
    Nq, Nk, causal = case
    run_full(720 + Nq % 97, 1, Nq, Nk, 4, 1, 64, "f16", causal, window=(40, 25))


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_window_head_dims(d):
    run_full(730 + HEAD_DIMS.index(d), 1, 260, 260, 2, 1, d, "bf16", False, window=(70, 10))


def test_window_oracle_forward_inputs():
    run_full(740, 1, 300, 300, 2, 2, 128, "bf16", False, fwd="oracle", window=(50, 50))


def test_window_open_band_equals_plain():
    """(-1, -1) through attention_backward takes fa_bwd; a band wider than the
    sequence through fa_bwd_window must give the same bits."""
    import torch
    qb, kb, vb, dob = inputs(741, 1, 300, 300, 4, 2, 128, "bf16")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (qb, kb, vb, dob))
    o, lse = attention(qd, kd, vd)
    plain = attention_backward(qd, kd, vd, o, lse, dod)
    wide = attention_backward(qd, kd, vd, o, lse, dod, window=(100000, 100000))
    for a, b in zip(plain, wide):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["bwd_bf16_4096_full", "bwd_bf16_4096_causal"])
def test_benchmark_shape_whole_heads(name):
    """The benchmark workload on the GPU; whole (b, h) heads of the first and the last
    batch element against the oracle (every head is independent here: Hq = Hkv), under the
element-wise bound and the pages' twice-the-baseline rule."""
    w = synthetic.WORKLOADS[name]
    q, k, v = w.inputs()
    do = w.grad_out()
    print(f"[bwd] {w.name}", flush=True)
    qd, kd, vd, dod = (to_dev(x, w.dtype) for x in (q, k, v, do))
    o, lse = attention(qd, kd, vd, causal=w.causal, scale=w.scale)
    dq, dk, dv = attention_backward(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale)
    assert w.Hq == w.Hkv
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        args = [oracle.widen(x[sl], w.dtype) for x in (q, k, v, do)]
        ref = oracle.backward(*args, causal=w.causal, scale=w.scale)
        mag = oracle.backward_magnitudes(*args, causal=w.causal, scale=w.scale)
        flo = oracle.backward_operand_sums(args[0], args[1], args[3], causal=w.causal, scale=w.scale)
        base = cmp.emulate_backward(*args, w.causal, w.scale, w.dtype)
        for g, r, m, f, e, n in zip((dq, dk, dv), ref, mag, flo, base, ("dq", "dk", "dv")):
            got = to_np(g[sl])
            worst = cmp.check_grad(got, r, m, w.dtype, f"{w.name} b={b} h={h} {n}", floor=f)
            eg, eb = cmp.check_grad_vs_baseline(got, r, e, w.dtype, f"{w.name} b={b} h={h} {n} vs float32 baseline")
            print(f"[bwd] {w.name} b={b} h={h} {n}: ratio {worst:.3g}, max error {eg:.3g} (baseline {eb:.3g})",
                  flush=True)
