"""GPU parity of fa_bwd_varlen (backward over a packed variable-length batch)
against the fp64 oracle, through the C ABI. Packing is an indexing convention,
so sequence b's gradients must equal the plain backward of its own query and
key rows (oracle.backward on that sequence alone), under the element-wise
rounding bound of _compare.check_grad. O and LSE come from fa_fwd_varlen."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import device, to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import (attention, attention_backward, attention_varlen,  # noqa: E402
                                          attention_varlen_backward)


def packed(wid, lq, lk, Hq, Hkv, d, dtype):
    tq, tk = int(sum(lq)), int(sum(lk))
    qb = synthetic.normal_bits(wid, synthetic.Q_ID, (1, tq, Hq, d), dtype)[0]
    kb = synthetic.normal_bits(wid, synthetic.K_ID, (1, tk, Hkv, d), dtype)[0]
    vb = synthetic.normal_bits(wid, synthetic.V_ID, (1, tk, Hkv, d), dtype)[0]
    dob = synthetic.normal_bits(wid, synthetic.DO_ID, (1, tq, Hq, d), dtype)[0]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    return qb, kb, vb, dob, cq, ck


def run(wid, lq, lk, Hq, Hkv, d, dtype, causal=False):
    import torch
    qb, kb, vb, dob, cq, ck = packed(wid, lq, lk, Hq, Hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    print(f"[bwd varlen] wid={wid} lq={list(lq)} lk={list(lk)} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}",
          flush=True)
    dev = device()
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (qb, kb, vb, dob))
    cqd, ckd = torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev)
    mq, mk = max(max(lq), 1), max(max(lk), 1)
    o, lse = attention_varlen(qd, kd, vd, cqd, ckd, mq, causal=causal, scale=scale)
    # rows outside every sequence are not written: start from zeros to compare them too
    dq, dk, dv = torch.zeros_like(qd), torch.zeros_like(kd), torch.zeros_like(vd)
    attention_varlen_backward(qd, kd, vd, o, lse, dod, cqd, ckd, mq, mk, causal=causal, scale=scale,
                              dq=dq, dk=dk, dv=dv)
    dq, dk, dv = to_np(dq), to_np(dk), to_np(dv)
    worst = 0.0
    for b in range(len(lq)):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        what = f"seq {b} (nq={q1 - q0}, nk={k1 - k0}, causal={causal}, d={d})"
        if q1 == q0:
            continue   # no query row: its key rows get zero gradients, checked below
        if k1 == k0:   # no key: the query rows get dQ = 0
            assert np.all(dq[q0:q1] == 0), what
            continue
        args = [oracle.widen(x[None, r0:r1], dtype) for x, r0, r1 in
                ((qb, q0, q1), (kb, k0, k1), (vb, k0, k1), (dob, q0, q1))]
        ref = oracle.backward(*args, causal=causal, scale=scale)
        mag = oracle.backward_magnitudes(*args, causal=causal, scale=scale)
        flo = oracle.backward_operand_sums(args[0], args[1], args[3], causal=causal, scale=scale)
        for g, r, m, f, n in zip((dq[None, q0:q1], dk[None, k0:k1], dv[None, k0:k1]), ref, mag, flo,
                                 ("dq", "dk", "dv")):
            if g.size:
                worst = max(worst, cmp.check_grad(g, r, m, dtype, f"{what} {n}", floor=f))
    for b in range(len(lq)):
        if cq[b + 1] == cq[b]:   # keys no query sees have zero gradients
            assert np.all(dk[ck[b]:ck[b + 1]] == 0) and np.all(dv[ck[b]:ck[b + 1]] == 0)
    print(f"[bwd varlen] worst ratio to u*M: {worst:.3g}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_self_attention(causal):
    lens = [1000, 1, 300, 0, 129, 256]
    run(3500 + causal, lens, lens, 8, 2, 128, "bf16", causal)


@pytest.mark.parametrize("causal", [False, True])
def test_queries_and_keys_differ_per_sequence(causal):
    # bottom-right per sequence; a sequence without keys gets dQ = 0 and no dK, dV rows
    run(3600 + causal, [50, 200, 7, 64], [300, 10, 0, 64], 8, 8, 64, "f16", causal)


@pytest.mark.parametrize("causal", [False, True])
def test_many_short_sequences(causal):
    # 600 sequences of 0 to 24 rows (seeded): the grid is mostly workgroups past
    # their sequence's end, which must exit cleanly
    lens = [int(x) for x in np.random.default_rng(3650).integers(0, 25, size=600)]
    run(3650 + causal, lens, lens, 4, 2, 64, "bf16", causal)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 192, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_dims(d, dtype):
    run(3700 + d + (dtype == "bf16"), [130, 5, 77], [130, 40, 77], 4, 2, d, dtype, causal=(d % 64 == 0))


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_the_dense_backward(causal):
    """[B][N] packed rows are the dense layout: the same gradients bit for bit."""
    import torch
    B, N, Hq, Hkv, d = 3, 384, 8, 4, 128
    qb, kb, vb, dob, cq, ck = packed(3800 + causal, [N] * B, [N] * B, Hq, Hkv, d, "bf16")
    dev = device()
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (qb, kb, vb, dob))
    o, lse = attention_varlen(qd, kd, vd, torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev), N,
                              causal=causal)
    packed_grads = attention_varlen_backward(qd, kd, vd, o, lse, dod, torch.from_numpy(cq).to(dev),
                                             torch.from_numpy(ck).to(dev), N, N, causal=causal)
    shape_q, shape_k = (B, N, Hq, d), (B, N, Hkv, d)
    o_d, lse_d = attention(qd.view(shape_q), kd.view(shape_k), vd.view(shape_k), causal=causal)
    dense = attention_backward(qd.view(shape_q), kd.view(shape_k), vd.view(shape_k), o_d, lse_d,
                               dod.view(shape_q), causal=causal)
    for a, b in zip(packed_grads, dense):
        assert torch.equal(a.reshape(b.shape).view(torch.int16), b.view(torch.int16))
