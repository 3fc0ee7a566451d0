"""GPU checks beyond parity: bitwise repeatability (the forward pass is
deterministic, "flash-attention-v100" README, flash_attn_func docstring),
outputs fully overwritten, and no write outside the output and workspace
buffers (canaries)."""
import numpy as np
import pytest

import synthetic
from gpu_util import device, to_dev

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention, decode, decode_workspace_bytes  # noqa: E402


def qkv(wid, B, Nq, Nk, Hq, Hkv, d, dtype):
    return (to_dev(synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype), dtype),
            to_dev(synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), dtype), dtype),
            to_dev(synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), dtype), dtype))


@pytest.mark.parametrize("causal", [False, True])
def test_forward_is_bitwise_deterministic(causal):
    import torch
    q, k, v = qkv(1000, 2, 1000, 1000, 8, 4, 128, "f16")
    o1, l1 = attention(q, k, v, causal=causal)
    o2, l2 = attention(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_decode_is_bitwise_deterministic():
    import torch
    q, k, v = qkv(1001, 4, 8, 3000, 32, 8, 128, "bf16")
    o1, l1 = decode(q, k, v, num_splits=16)
    o2, l2 = decode(q, k, v, num_splits=16)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def canary_view(n_elems, dtype, pad=4096):
    """A view of n_elems in the middle of a buffer whose borders hold a sentinel."""
    import torch
    buf = torch.full((n_elems + 2 * pad,), float("nan"), dtype=dtype, device=device())
    buf[:pad] = 7.0
    buf[pad + n_elems:] = 7.0
    return buf, buf[pad:pad + n_elems], pad


def test_forward_writes_every_output_and_nothing_else():
    import torch
    B, Nq, Nk, Hq, Hkv, d = 2, 333, 200, 6, 3, 64
    q, k, v = qkv(1002, B, Nq, Nk, Hq, Hkv, d, "bf16")
    obuf, o, pad = canary_view(B * Nq * Hq * d, torch.bfloat16)
    lbuf, lse, lpad = canary_view(B * Hq * Nq, torch.float32)
    attention(q, k, v, causal=True, out=o.view(B, Nq, Hq, d), lse=lse.view(B, Hq, Nq))
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    assert not torch.isnan(lse).any()          # fully masked rows are -inf, never NaN
    assert torch.all(obuf[:pad] == 7) and torch.all(obuf[pad + o.numel():] == 7)
    assert torch.all(lbuf[:lpad] == 7) and torch.all(lbuf[lpad + lse.numel():] == 7)


def test_decode_writes_every_output_and_stays_in_workspace():
    import torch
    B, Nq, Nk, Hq, Hkv, d, S = 3, 2, 1111, 8, 2, 128, 7
    q, k, v = qkv(1003, B, Nq, Nk, Hq, Hkv, d, "f16")
    need = decode_workspace_bytes(B, Nq, Hq, d, S)
    wbuf = torch.full((need + 8192,), 0x5A, dtype=torch.uint8, device=device())
    ws = wbuf[4096:4096 + need]
    obuf, o, pad = canary_view(B * Nq * Hq * d, torch.float16)
    decode(q, k, v, num_splits=S, workspace=ws, out=o.view(B, Nq, Hq, d))
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    assert torch.all(obuf[:pad] == 7) and torch.all(obuf[pad + o.numel():] == 7)
    assert torch.all(wbuf[:4096] == 0x5A) and torch.all(wbuf[4096 + need:] == 0x5A)
