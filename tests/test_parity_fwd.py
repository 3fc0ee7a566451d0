"""GPU parity of fa_fwd against the fp64 oracle, through the C ABI.

Whole tensors at small sizes (several tiles, ragged tails, every head dim,
both dtypes, Nq != Nk, fully masked rows) and at the pages' headline shape
for one batch element; sampled rows (all heads, first and last batch) at the
long-sequence and GQA sizes, in the launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import oracle_rows, to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention  # noqa: E402

HEAD_DIMS = (32, 64, 96, 128, 192, 256)


def run_full(wid, B, Nq, Nk, Hq, Hkv, d, dtype, causal, qk_mult=1.0, scale=None):
    sq, sk = (B, Nq, Hq, d), (B, Nk, Hkv, d)
    qb = synthetic.normal_bits(wid, 0, sq, dtype, qk_mult)
    kb = synthetic.normal_bits(wid, 1, sk, dtype, qk_mult)
    vb = synthetic.normal_bits(wid, 2, sk, dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    print(f"[fwd] wid={wid} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}", flush=True)
    o, lse = attention(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), causal=causal, scale=scale)
    o_ref, lse_ref = oracle.attention_bits(qb, kb, vb, dtype, causal=causal, scale=scale)
    what = f"B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}"
    stats = cmp.check_o(to_np(o), o_ref, dtype, what)
    cmp.check_lse(to_np(lse), lse_ref, what)
    return stats


def test_tiny_workload():
    w = synthetic.WORKLOADS["tiny_f16_128"]
    run_full(w.wid, w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.causal)


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
    (1, 3, 65537, 2, 1, 128, "f16", False),   # a few rows over 65537 keys (2049 tiles, ragged tail)
    (1, 3, 65537, 2, 1, 128, "bf16", True),
    (1, 70001, 3, 2, 2, 128, "f16", False),   # 70001 rows (the 256-row shape) over 3 keys
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes(case):
    run_full(100 + EDGE.index(case), *case)


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims(d, dtype, causal):
    wid = 200 + HEAD_DIMS.index(d) * 4 + (dtype == "bf16") * 2 + int(causal)
    run_full(wid, 2, 200, 333, 6, 2, d, dtype, causal)


def ramp_bits(wid, tensor_id, shape, dtype, lo, hi):
    """N(0,1) samples whose rows along the sequence axis are scaled from lo up to hi,
    rounded to dtype: scores then grow along the keys, so the running max of every
    row keeps rising tile after tile."""
    rng = np.random.default_rng([wid, tensor_id])
    x = rng.standard_normal(shape, dtype=np.float32)
    ramp = np.linspace(lo, hi, shape[1], dtype=np.float32)[None, :, None, None]
    return synthetic.to_bits(x * ramp, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_moves_in_unmasked_tiles(dtype, causal):
    """Keys scaled up along the sequence (x0.2 to x4, scale 0.5): a row's scores rise
    by far more than 2^14 in log2 units across the unmasked tiles, so the reference
    max is moved in the middle of the key loop (a lane's sum of probabilities
    exceeds the cap and the tile is redone against its own max), not only on the
    first tile."""
    B, N, H, d = 1, 1024, 4, 128
    qb = synthetic.normal_bits(91, 0, (B, N, H, d), dtype)
    kb = ramp_bits(91, 1, (B, N, H, d), dtype, 0.2, 4.0)
    vb = synthetic.normal_bits(91, 2, (B, N, H, d), dtype)
    print(f"[fwd rebase] {dtype} causal={causal}", flush=True)
    o, lse = attention(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), causal=causal, scale=0.5)
    o_ref, lse_ref = oracle.attention_bits(qb, kb, vb, dtype, causal=causal, scale=0.5)
    what = f"rising scores {dtype} causal={causal}"
    cmp.check_o(to_np(o), o_ref, dtype, what)
    cmp.check_lse(to_np(lse), lse_ref, what)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_grouped_heads_order(causal, dtype, d):
    """32 (batch, head) pairs with 4 query heads per KV head and a ragged query
    count: the work orders keep a KV group's query heads on one XCD (a permutation
    used only when the pair count is a multiple of 8 groups)."""
    run_full(96, 2, 300, 300, 16, 4, d, dtype, causal)


def test_scale_is_used_as_passed():
    run_full(300, 1, 130, 130, 2, 2, 64, "f16", False, scale=0.37)
    run_full(301, 1, 130, 130, 2, 2, 64, "bf16", True, scale=0.0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,scale", [(64, -1.0), (128, "-1/sqrt(d)"), (256, "-1/sqrt(d)")])
def test_negative_scale(dtype, causal, d, scale):
    """O and LSE at a negative scale (the softmax of -|scale| q.k; the kernel flips
    the sign of Q and uses |scale|), several tiles and ragged tails, GQA heads."""
    sc = -1.0 if scale == -1.0 else -1.0 / math.sqrt(d)
    run_full(320 + 4 * (d // 64) + 2 * (dtype == "bf16") + int(causal), 2, 300, 333, 6, 2, d, dtype, causal,
             scale=sc)


def run_sampled(w, seed):
    """Whole workload on the GPU; oracle on sampled rows of b = 0 and b = B-1."""
    q, k, v = w.inputs()
    print(f"[fwd sampled] {w.name}", flush=True)
    o, lse = attention(to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), causal=w.causal, scale=w.scale)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    del o, lse
    rng = np.random.default_rng(seed)
    rows = cmp.sample_rows(w.Nq, rng)
    worst = {}
    for b in sorted({0, w.B - 1}):
        o_ref, lse_ref = oracle_rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], w.dtype, rows, w.causal, w.scale)
        what = f"{w.name} b={b}"
        st = cmp.check_o(o_np[b:b + 1, rows].astype(np.float64), o_ref, w.dtype, what)
        cmp.check_lse(lse_np[b:b + 1][:, :, rows].astype(np.float64), lse_ref, what)
        # secondary rule: within 2x the error of a plain float32 implementation (+1 ulp)
        qf, kf, vf = (oracle.widen(x[b], w.dtype) for x in (q, k, v))
        for h in (0, w.Hq - 1):
            g = h // (w.Hq // w.Hkv)
            base = cmp.emulate_rows(qf[:, h], kf[:, g], vf[:, g], rows, h, w.causal, w.scale, w.dtype, w.Nq)
            ref = o_ref[0, :, h]
            e_gpu = np.abs(o_np[b, rows, h] - ref).max()
            e_base = np.abs(base - ref).max()
            slack = cmp.ulp(np.abs(ref).max(), w.dtype)
            assert e_gpu <= 2 * e_base + slack, f"{what} h={h}: {e_gpu:.3g} > 2*{e_base:.3g} + {slack:.3g}"
        worst = {k2: max(worst.get(k2, 0), v2) for k2, v2 in st.items()}
    print(f"[fwd sampled] {w.name}: {cmp.fmt(worst)}", flush=True)


def test_headline_whole_workload():
    """The pages' headline workload [16, 1024, 32, 128] f16 run once on the GPU in the
    benchmark's launch configuration and compared with the oracle on every element of
    every batch; then the secondary rule on sampled rows of the first and last batch."""
    w = synthetic.WORKLOADS["headline_f16_1024"]
    q, k, v = w.inputs()
    print(f"[fwd] {w.name} whole", flush=True)
    o, lse = attention(to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype), causal=False, scale=w.scale)
    o_np, lse_np = to_np(o), to_np(lse)
    del o, lse
    o_ref, lse_ref = oracle.attention_bits(q, k, v, w.dtype, scale=w.scale)
    st = cmp.check_o(o_np, o_ref, w.dtype, "headline whole")
    cmp.check_lse(lse_np, lse_ref, "headline whole")
    print(f"[fwd] {w.name} whole: {cmp.fmt(st)}", flush=True)
    del o_np, o_ref
    run_sampled(w, 7)


LONG = [n for n in synthetic.WORKLOADS if n.startswith("long_")]
GQA = [n for n in synthetic.WORKLOADS if n.startswith("gqa_")]


@pytest.mark.parametrize("name", LONG)
def test_long_sequence_sampled(name):
    run_sampled(synthetic.WORKLOADS[name], 11)


@pytest.mark.parametrize("name", GQA)
def test_gqa_head_dim_sweep_sampled(name):
    run_sampled(synthetic.WORKLOADS[name], 13)


@pytest.mark.parametrize("case", [(1, 3100, 700, 4, 2, None), (1, 3072, 3073, 2, 1, -0.05), (2, 4097, 300, 2, 2, None),
                                  (1, 3072, 17, 2, 2, None), (1, 3333, 64, 2, 1, None)],
                         ids=lambda c: "x".join(map(str, c)))
def test_wide_workgroups(case):
    """fp16, d = 128, no mask, 3072 query rows or more: the eight-wave, 256-row
    workgroup shape (64-key tiles). Whole tensors with a partial last row tile,
    ragged key counts (also fewer keys than one tile, and exactly one tile),
    grouped heads and a negative scale."""
    B, nq, nk, hq, hkv, scale = case
    run_full(7000 + nq % 97 + nk % 89, B, nq, nk, hq, hkv, 128, "f16", False, scale=scale)


def test_wide_workgroups_rebase():
    """Rising scores (as in test_reference_moves_in_unmasked_tiles) in the wide shape."""
    B, N, H, d = 1, 3072, 2, 128
    qb = synthetic.normal_bits(92, 0, (B, N, H, d), "f16")
    kb = ramp_bits(92, 1, (B, N, H, d), "f16", 0.2, 4.0)
    vb = synthetic.normal_bits(92, 2, (B, N, H, d), "f16")
    o, lse = attention(to_dev(qb, "f16"), to_dev(kb, "f16"), to_dev(vb, "f16"), scale=0.5)
    o_ref, lse_ref = oracle.attention_bits(qb, kb, vb, "f16", scale=0.5)
    cmp.check_o(to_np(o), o_ref, "f16", "wide rising scores")
    cmp.check_lse(to_np(lse), lse_ref, "wide rising scores")
