"""GPU parity of fa_decode_splitkv_paged against the fp64 oracle, through the C ABI.

The paged cache is the one of flash_attn_with_kvcache ("flash-attention-v100"
README, How to use FlashAttention: block_table and cache_seqlens): the test
gathers each sequence's pages into a contiguous cache on the host and gives the
oracle the per-sequence lengths, so the oracle never sees pages."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import device, to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import decode, decode_paged  # noqa: E402


def paged_case(wid, B, Nq, Hq, Hkv, d, dtype, page_size, max_pages, lens, extra_pages=3):
    num_pages = B * max_pages + extra_pages
    qb = synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype)
    kp = synthetic.normal_bits(wid, 1, (num_pages, page_size, Hkv, d), dtype)
    vp = synthetic.normal_bits(wid, 2, (num_pages, page_size, Hkv, d), dtype)
    bt = synthetic.block_table(wid, B, max_pages, num_pages)
    lens = np.asarray(lens, np.int32)
    return qb, kp, vp, bt, lens


def gathered(pool_bits, bt, page_size):
    """[B, max_pages * page_size, Hkv, d]: each sequence's pages in logical order."""
    B, P = bt.shape
    return pool_bits[bt.reshape(-1)].reshape(B, P * page_size, *pool_bits.shape[2:])


def run(wid, B, Nq, Hq, Hkv, d, dtype, page_size, max_pages, lens, splits=16, causal=False, scale=None):
    import torch
    qb, kp, vp, bt, lens = paged_case(wid, B, Nq, Hq, Hkv, d, dtype, page_size, max_pages, lens)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    print(f"[paged] wid={wid} B={B} Nq={Nq} Hq={Hq} Hkv={Hkv} d={d} {dtype} page={page_size} "
          f"max_pages={max_pages} lens={lens.tolist()} S={splits} causal={causal} scale={scale}", flush=True)
    dev = device()
    o, lse = decode_paged(to_dev(qb, dtype), to_dev(kp, dtype), to_dev(vp, dtype),
                          torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev),
                          num_splits=splits, causal=causal, scale=scale)
    ref = oracle.attention_bits(qb, gathered(kp, bt, page_size), gathered(vp, bt, page_size), dtype,
                                causal=causal, scale=scale, seqlens_k=lens)
    what = f"paged page={page_size} lens={lens.tolist()} S={splits} causal={causal} d={d} scale={scale}"
    st = cmp.check_o(to_np(o), ref[0], dtype, what)
    cmp.check_lse(to_np(lse), ref[1], what)
    return st, to_np(o), to_np(lse)


def test_paged_decode_workload_shape():
    # decode workload geometry (Hq 32, Hkv 8, d 128, bf16) with 256-key pages and ragged lengths
    st, _, _ = run(2000, 4, 1, 32, 8, 128, "bf16", 256, 32, [8192, 5000, 257, 1])
    print(f"[paged] workload shape: {cmp.fmt(st)}", flush=True)


@pytest.mark.parametrize("page_size", [32, 64, 256, 1024])
def test_page_sizes(page_size):
    max_pages = max(1, 2048 // page_size)
    run(2100 + page_size, 3, 2, 8, 2, 128, "bf16", page_size, max_pages, [2048, 1000, 33])


def test_empty_and_tiny_sequences():
    # a sequence with no key gets O = 0 and LSE = -inf; lengths below one tile
    st, o, lse = run(2200, 4, 1, 8, 2, 64, "f16", 64, 4, [0, 1, 31, 256], splits=8)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("splits", [1, 3, 16, 64])
def test_split_counts(splits):
    run(2300 + splits, 2, 1, 16, 4, 128, "bf16", 128, 12, [1536, 700], splits=splits)


@pytest.mark.parametrize("Nq,lens", [(4, [1024, 3, 600]), (8, [8, 5, 2048])])
def test_causal_aligned_to_each_sequence(Nq, lens):
    # bottom-right per sequence: rows with i + len - Nq < 0 see no key
    run(2400 + Nq, 3, Nq, 8, 2, 128, "bf16", 256, 8, lens, causal=True)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 192, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_dims(d, dtype):
    run(2500 + d + (dtype == "bf16"), 2, 2, 8, 2, d, dtype, 64, 10, [640, 333], splits=5)


def test_contiguous_cache_as_one_page_per_sequence():
    # a contiguous [B][Nk][Hkv][d] cache is the pool with page_size = Nk and block_table[b] = b:
    # the paged entry point must then give the contiguous one's result bit for bit
    import torch
    wid, B, Nq, Nk, Hq, Hkv, d = 2600, 3, 2, 1024, 16, 4, 128
    qb = synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), "bf16")
    kb = synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), "bf16")
    vb = synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), "bf16")
    q, k, v = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    dev = device()
    bt = torch.arange(B, dtype=torch.int32, device=dev).reshape(B, 1)
    lens = torch.full((B,), Nk, dtype=torch.int32, device=dev)
    o1, l1 = decode(q, k, v, num_splits=16)
    o2, l2 = decode_paged(q, k, v, bt, lens, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_out_of_range_page_reads_zeros_without_leaving_the_pool():
    # sequence 1's table points outside the pool; the call completes and the
    # other sequences are unaffected
    import torch
    wid, B, Nq, Hq, Hkv, d, ps, mp = 2700, 3, 1, 8, 2, 128, 64, 4
    qb, kp, vp, bt, lens = paged_case(wid, B, Nq, Hq, Hkv, d, "bf16", ps, mp, [256, 256, 200])
    bad = bt.copy()
    bad[1, 2] = 1 << 30
    bad[1, 3] = -5
    dev = device()
    o, lse = decode_paged(to_dev(qb, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                          torch.from_numpy(bad).to(dev), torch.from_numpy(lens).to(dev), num_splits=4)
    torch.cuda.synchronize()
    ref = oracle.attention_bits(qb, gathered(kp, bt, ps), gathered(vp, bt, ps), "bf16",
                                scale=1.0 / math.sqrt(d), seqlens_k=lens)
    for b in (0, 2):
        cmp.check_o(to_np(o)[b:b + 1], ref[0][b:b + 1], "bf16", f"seq {b}")
        cmp.check_lse(to_np(lse)[b:b + 1], ref[1][b:b + 1], f"seq {b}")
    assert np.all(np.isfinite(to_np(o)[1]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [-1.0, -0.125])
def test_paged_negative_scale(dtype, scale):
    """A negative scale over a paged cache (d = 64, so -0.125 is -1/sqrt(d)), causal
    with ragged lengths: the oracle decides."""
    run(2300 + (dtype == "bf16") + 2 * (scale == -1.0), 3, 2, 8, 2, 64, dtype, 64, 12, [700, 64, 333],
        splits=8, causal=True, scale=scale)
