"""CPU pins of the output tolerance rule (tests/_compare.check_o): the correctly
rounded exact result passes it, and results with a plausible mistake fail it."""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic


def _round(x, dtype):
    import torch
    t = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(x)).to(t).to(torch.float64).numpy()


def _case(nk, dtype, wid=6490):
    q = synthetic.normal_bits(wid, 0, (1, 3, 4, 128), dtype)
    k = synthetic.normal_bits(wid, 1, (1, nk, 4, 128), dtype)
    v = synthetic.normal_bits(wid, 2, (1, nk, 4, 128), dtype)
    o, _ = oracle.attention_bits(q, k, v, dtype, scale=1.0 / math.sqrt(128))
    return q, k, v, o


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nk", [2, 300])
def test_correctly_rounded_result_passes(dtype, nk):
    # with two keys |O| is near 1 and bf16 rounding alone is close to 1e-3 on average
    _, _, _, o = _case(nk, dtype)
    cmp.check_o(_round(o, dtype), o, dtype, "rounded exact result")


def test_one_ulp_bias_fails():
    # every bf16 element one ulp high (2^-8 near |O| = 0.65): half an ulp of excess
    # everywhere, above 1e-3 on average
    _, _, _, o = _case(2, "bf16")
    biased = _round(o, "bf16") + cmp.ulp(o, "bf16")
    with pytest.raises(AssertionError):
        cmp.check_o(biased, o, "bf16", "biased")


@pytest.mark.parametrize("mistake", ["no_scale", "key_dropped", "rows_swapped"])
def test_planted_mistakes_fail(mistake):
    q, k, v, o = _case(300, "bf16")
    if mistake == "no_scale":
        bad, _ = oracle.attention_bits(q, k, v, "bf16", scale=1.0)
    elif mistake == "key_dropped":
        bad, _ = oracle.attention_bits(q, k[:, 1:], v[:, 1:], "bf16", scale=1.0 / math.sqrt(128))
    else:
        bad = o[:, [1, 0, 2]]
    with pytest.raises(AssertionError):
        cmp.check_o(_round(bad, "bf16"), o, "bf16", mistake)
