"""GPU parity of fa_fwd_window (sliding-window local attention) against the fp64
oracle, through the C ABI ("flash-attention-v100" README, How to use
FlashAttention: window_size, the band aligned bottom-right like the causal mask)."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention  # noqa: E402


def inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype):
    return (synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype),
            synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), dtype),
            synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), dtype))


def run(wid, B, Nq, Nk, Hq, Hkv, d, dtype, window, causal=False):
    qb, kb, vb = inputs(wid, B, Nq, Nk, Hq, Hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    print(f"[window] wid={wid} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} window={window} "
          f"causal={causal}", flush=True)
    o, lse = attention(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), causal=causal, scale=scale,
                       window=window)
    ref = oracle.attention_bits(qb, kb, vb, dtype, causal=causal, scale=scale, window=window)
    what = f"window={window} causal={causal} Nq={Nq} Nk={Nk} d={d}"
    st = cmp.check_o(to_np(o), ref[0], dtype, what)
    cmp.check_lse(to_np(lse), ref[1], what)
    return st


@pytest.mark.parametrize("window", [(0, 0), (16, 0), (100, 100), (-1, 50), (300, -1), (0, -1), (63, 64),
                                    (1000, 1000)])
def test_bands(window):
    run(4000 + sum(window) % 97, 2, 700, 700, 8, 2, 128, "bf16", window)


@pytest.mark.parametrize("Nq,Nk", [(300, 1000), (1000, 300), (129, 257)])
def test_bottom_right_alignment(Nq, Nk):
    # Nq > Nk leaves early rows with no key (O = 0, LSE = -inf)
    run(4100 + Nq % 89, 2, Nq, Nk, 8, 8, 64, "f16", (40, 3))


def test_causal_fixes_the_right_edge():
    run(4200, 2, 500, 500, 8, 2, 128, "bf16", (64, 7), causal=True)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 192, 256])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_head_dims(d, dtype):
    run(4300 + d + (dtype == "bf16"), 1, 333, 333, 4, 2, d, dtype, (70, 20))


def test_long_local_causal():
    # a 4096-token sequence with a 256-key causal window: most tiles are skipped
    st = run(4400, 1, 4096, 4096, 4, 4, 128, "bf16", (256, 0))
    print(f"[window] long local causal: {cmp.fmt(st)}", flush=True)


def test_open_band_equals_the_plain_and_causal_calls():
    import torch
    qb, kb, vb = inputs(4500, 2, 640, 640, 8, 2, 128, "f16")
    q, k, v = to_dev(qb, "f16"), to_dev(kb, "f16"), to_dev(vb, "f16")
    o1, l1 = attention(q, k, v)
    o2, l2 = attention(q, k, v, window=(-1, -1))
    o3, l3 = attention(q, k, v, causal=True)
    o4, l4 = attention(q, k, v, window=(-1, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
