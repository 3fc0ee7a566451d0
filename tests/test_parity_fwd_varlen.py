"""GPU parity of fa_fwd_varlen (packed variable-length batch) against the fp64
oracle, through the C ABI. The oracle sees each sequence on its own: packing is
an indexing convention, so sequence b's result must equal plain attention over
its own query and key rows ("flash-attention-v100" README, Changelog 2.0 names
the varlen entry point; the prefix-sum reading is documented in include/fa.h)."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import device, to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention, attention_varlen  # noqa: E402


def packed(wid, lq, lk, Hq, Hkv, d, dtype):
    tq, tk = int(sum(lq)), int(sum(lk))
    qb = synthetic.normal_bits(wid, 0, (1, tq, Hq, d), dtype)[0]
    kb = synthetic.normal_bits(wid, 1, (1, tk, Hkv, d), dtype)[0]
    vb = synthetic.normal_bits(wid, 2, (1, tk, Hkv, d), dtype)[0]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    return qb, kb, vb, cq, ck


def run(wid, lq, lk, Hq, Hkv, d, dtype, causal=False):
    import torch
    qb, kb, vb, cq, ck = packed(wid, lq, lk, Hq, Hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    print(f"[varlen] wid={wid} lq={list(lq)} lk={list(lk)} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}",
          flush=True)
    dev = device()
    o, lse = attention_varlen(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype),
                              torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev), max(max(lq), 1),
                              causal=causal, scale=scale)
    o, lse = to_np(o), to_np(lse)
    stats = []
    for b in range(len(lq)):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1 == q0:
            continue
        what = f"seq {b} (nq={q1 - q0}, nk={k1 - k0}, causal={causal}, d={d})"
        if k1 == k0:   # no key: O = 0, LSE = -inf
            assert np.all(o[q0:q1] == 0) and np.all(np.isneginf(lse[:, q0:q1])), what
            continue
        ro, rl = oracle.attention_bits(qb[None, q0:q1], kb[None, k0:k1], vb[None, k0:k1], dtype,
                                       causal=causal, scale=scale)
        stats.append(cmp.check_o(o[None, q0:q1], ro, dtype, what))
        cmp.check_lse(lse[None, :, q0:q1], rl, what)
    return stats


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_self_attention(causal):
    lens = [1000, 1, 300, 0, 129, 256]
    run(3000 + causal, lens, lens, 8, 2, 128, "bf16", causal)


@pytest.mark.parametrize("causal", [False, True])
def test_queries_and_keys_differ_per_sequence(causal):
    # bottom-right per sequence; a sequence without keys gives O = 0, LSE = -inf
    run(3100 + causal, [50, 200, 7, 64], [300, 10, 0, 64], 8, 8, 64, "f16", causal)


@pytest.mark.parametrize("causal", [False, True])
def test_many_short_sequences(causal):
    # 600 sequences of 0 to 24 rows (seeded): the grid is mostly workgroups past
    # their sequence's end, which must exit cleanly
    lens = [int(x) for x in np.random.default_rng(3150).integers(0, 25, size=600)]
    run(3150 + causal, lens, lens, 4, 2, 64, "bf16", causal)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 192, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_dims(d, dtype):
    run(3200 + d + (dtype == "bf16"), [130, 5, 77], [130, 40, 77], 4, 2, d, dtype, causal=(d % 64 == 0))


def test_equal_lengths_match_the_dense_kernel():
    # [B][N] packed rows are the dense layout: O bit for bit, LSE transposed [Hq][B*N] vs [B][Hq][N]
    import torch
    B, N, Hq, Hkv, d = 3, 384, 8, 4, 128
    qb, kb, vb, cq, ck = packed(3300, [N] * B, [N] * B, Hq, Hkv, d, "f16")
    dev = device()
    q, k, v = to_dev(qb, "f16"), to_dev(kb, "f16"), to_dev(vb, "f16")
    o1, l1 = attention(q.view(B, N, Hq, d), k.view(B, N, Hkv, d), v.view(B, N, Hkv, d), causal=True)
    o2, l2 = attention_varlen(q, k, v, torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev), N,
                              causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(B * N, Hq, d), o2)
    assert torch.equal(l1.permute(1, 0, 2).reshape(Hq, B * N), l2)


def test_malformed_prefix_sums_stay_inside_the_tensors():
    # decreasing and out-of-range entries are clamped into the tensors: the call
    # completes, the well-formed first sequence is exact, and sequence 1, whose
    # key range runs backwards, is empty (O = 0, LSE = -inf)
    import torch
    qb, kb, vb, cq, ck = packed(3400, [100, 50, 30], [100, 50, 30], 4, 2, 64, "bf16")
    bad_q = np.array([0, 100, 150, 1 << 30], np.int32)
    bad_k = np.array([0, 100, -7, 1 << 30], np.int32)
    dev = device()
    # validate=False: the binding's length check would refuse these tables before the library
    o, lse = attention_varlen(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"),
                              torch.from_numpy(bad_q).to(dev), torch.from_numpy(bad_k).to(dev), 200,
                              validate=False)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_bits(qb[None, :100], kb[None, :100], vb[None, :100], "bf16",
                                   scale=1.0 / math.sqrt(64))
    cmp.check_o(to_np(o)[None, :100], ro, "bf16", "seq 0")
    cmp.check_lse(to_np(lse)[None, :, :100], rl, "seq 0")
    assert np.all(to_np(o)[100:150] == 0) and np.all(np.isneginf(to_np(lse)[:, 100:150]))
