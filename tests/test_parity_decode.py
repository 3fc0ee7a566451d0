"""GPU parity of fa_decode_splitkv (split kernel + combine kernel) against the
fp64 oracle, through the C ABI. The oracle computes the unsplit definition, so
these tests also check that splitting and merging change nothing beyond
rounding (Flash-Decoding's split/LSE/combine steps)."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention, decode  # noqa: E402


def inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype):
    qb = synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype)
    kb = synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), dtype)
    vb = synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), dtype)
    return qb, kb, vb


def run(wid, B, Nq, Nk, Hq, Hkv, d, dtype, splits, causal=False, ref=None, scale=None):
    qb, kb, vb = inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    print(f"[decode] wid={wid} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} S={splits} "
          f"causal={causal} scale={scale}", flush=True)
    o, lse = decode(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), num_splits=splits,
                    causal=causal, scale=scale)
    if ref is None:
        ref = oracle.attention_bits(qb, kb, vb, dtype, causal=causal, scale=scale)
    what = f"decode B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} S={splits} causal={causal} scale={scale}"
    st = cmp.check_o(to_np(o), ref[0], dtype, what)
    cmp.check_lse(to_np(lse), ref[1], what)
    return st, ref, o


@pytest.mark.parametrize("name", ["decode_bf16_nq1", "decode_bf16_nq8"])
def test_decode_workloads(name):
    w = synthetic.WORKLOADS[name]
    st, _, _ = run(w.wid, w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.num_splits)
    print(f"[decode] {name}: {cmp.fmt(st)}", flush=True)


@pytest.mark.parametrize("splits", [1, 7, 16, 64, 256])
def test_split_count_invariance(splits):
    w = synthetic.WORKLOADS["decode_bf16_nq1"]
    run(w.wid, 2, 1, 2048, w.Hq, w.Hkv, w.d, w.dtype, splits)


@pytest.mark.parametrize("Nk,splits", [(1000, 16), (8191, 16), (33, 16), (1, 1), (31, 4), (100, 3), (300001, 64)])
def test_ragged_cache_lengths(Nk, splits):
    run(500 + Nk % 97, 2, 1, Nk, 8, 2, 128, "bf16", splits)


@pytest.mark.parametrize("Nq,Nk", [(8, 1024), (8, 5), (3, 700)])
def test_causal_decode_bottom_right(Nq, Nk):
    run(600 + Nq + Nk % 13, 2, Nq, Nk, 8, 2, 128, "bf16", 16, causal=True)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 192, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_dims(d, dtype):
    run(700 + d + (dtype == "bf16"), 2, 2, 777, 8, 2, d, dtype, 5)


def test_many_rows_per_group():
    # group 16 x Nq 4 = 64 rows per KV head: two 32-row blocks per chunk
    run(800, 2, 4, 1500, 32, 2, 128, "f16", 8)
    run(801, 1, 40, 600, 4, 4, 64, "bf16", 4, causal=True)


@pytest.mark.parametrize("case", [(5, 3, 6, 2, 96, "bf16", False), (3, 12, 8, 2, 64, "f16", False),
                                  (7, 12, 8, 2, 96, "bf16", True), (13, 1, 32, 8, 128, "bf16", False)],
                         ids=lambda c: "x".join(map(str, c)))
def test_odd_batch_and_row_blocks(case):
    """Batch counts that are not a multiple of the 8 XCDs (the batch is the
    split grid's fastest axis and the combine's), two 32-row blocks per KV head,
    and per-batch row counts that leave the combine's last workgroup partly idle."""
    B, Nq, Hq, Hkv, d, dtype, causal = case
    run(950 + B + Nq, B, Nq, 900, Hq, Hkv, d, dtype, 8, causal=causal)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [-1.0, "-1/sqrt(d)"])
def test_negative_scale(dtype, causal, scale):
    """A negative scale is used as passed: the softmax of -|scale| q.k. With
    scale = -1 at d = 64 the raw scores spread over tens of units, so a reference
    max taken from the unscaled scores would put probabilities far above the fp16
    range; the oracle decides."""
    d = 64
    sc = -1.0 / math.sqrt(d) if scale != -1.0 else -1.0
    run(1100 + (dtype == "bf16") + 2 * causal, 2, 3, 1500, 8, 2, d, dtype, 16, causal=causal, scale=sc)


def test_decode_matches_forward():
    wid, B, Nq, Nk, Hq, Hkv, d = 900, 2, 8, 4096, 32, 8, 128
    qb, kb, vb = inputs(wid, B, Nq, Nk, Hq, Hkv, d, "bf16")
    q, k, v = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    o1, l1 = decode(q, k, v, num_splits=16)
    o2, l2 = attention(q, k, v)
    ref = oracle.attention_bits(qb, kb, vb, "bf16")
    cmp.check_o(to_np(o1), ref[0], "bf16", "decode")
    cmp.check_o(to_np(o2), ref[0], "bf16", "fwd")
    assert float(np.abs(to_np(l1) - to_np(l2)).max()) <= 2e-3


@pytest.mark.parametrize("d", [192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_head_dims_row_blocks(d, causal, dtype):
    """The head dims whose split kernel loads each tile without running ahead
    (192) or shares it between two waves that own half of O's columns each
    (256): two 32-row blocks per KV head (group 8 x Nq 8), an odd batch, a
    ragged cache, the causal mask and a negative scale."""
    wid = 1200 + d + 2 * causal + (dtype == "bf16")
    run(wid, 3, 8, 1000, 16, 2, d, dtype, 7, causal=causal)
    run(wid + 10, 3, 8, 1000, 16, 2, d, dtype, 7, causal=causal, scale=-1.0 / math.sqrt(d))
