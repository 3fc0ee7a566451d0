"""GPU checks beyond parity: bitwise repeatability (the forward pass is
deterministic, "flash-attention-v100" README, flash_attn_func docstring; the
backward here has no atomics and is deterministic too),
outputs fully overwritten, and no write outside the output and workspace
buffers (canaries)."""
import numpy as np
import pytest

import synthetic
from gpu_util import device, to_dev

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import (attention, attention_backward, attention_varlen,  # noqa: E402
                                          attention_varlen_backward, bwd_workspace_bytes, decode,
                                          decode_workspace_bytes)


def qkv(wid, B, Nq, Nk, Hq, Hkv, d, dtype):
    return (to_dev(synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype), dtype),
            to_dev(synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), dtype), dtype),
            to_dev(synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), dtype), dtype))


@pytest.mark.parametrize("causal,nq", [(False, 1000), (True, 1000), (False, 3300)],
                         ids=["full", "causal", "wide"])
def test_forward_is_bitwise_deterministic(causal, nq):
    # nq = 3300 (fp16, d = 128, no mask) runs the 256-row workgroup shape
    import torch
    q, k, v = qkv(1000, 2, nq, 1000, 8, 4, 128, "f16")
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


@pytest.mark.parametrize("shape", [(2, 333, 200, 6, 3, 64, "bf16", True), (1, 3100, 130, 4, 2, 128, "f16", False)],
                         ids=["causal-d64", "wide-d128"])
def test_forward_writes_every_output_and_nothing_else(shape):
    # the second shape (fp16, d = 128, no mask, 3100 rows) runs the 256-row workgroups
    import torch
    B, Nq, Nk, Hq, Hkv, d, dtype, causal = shape
    q, k, v = qkv(1002, B, Nq, Nk, Hq, Hkv, d, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    obuf, o, pad = canary_view(B * Nq * Hq * d, tdt)
    lbuf, lse, lpad = canary_view(B * Hq * Nq, torch.float32)
    attention(q, k, v, causal=causal, out=o.view(B, Nq, Hq, d), lse=lse.view(B, Hq, Nq))
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


@pytest.mark.parametrize("window", [(-1, -1), (30, 10)])
def test_backward_writes_every_gradient_and_stays_in_workspace(window):
    """NaN-prefilled gradients are fully overwritten (rows that see no key get 0),
    and nothing is written around dQ, dK, dV or the workspace."""
    import torch
    B, Nq, Nk, Hq, Hkv, d = 2, 333, 200, 6, 3, 64
    q, k, v = qkv(1004, B, Nq, Nk, Hq, Hkv, d, "bf16")
    do = to_dev(synthetic.normal_bits(1004, synthetic.DO_ID, (B, Nq, Hq, d), "bf16"), "bf16")
    o, lse = attention(q, k, v, causal=True, window=window)
    need = bwd_workspace_bytes(B, Nq, Hq)
    wbuf = torch.full((need + 8192,), 0x5A, dtype=torch.uint8, device=device())
    ws = wbuf[4096:4096 + need]
    bufs = [canary_view(B * Nq * Hq * d, torch.bfloat16), canary_view(B * Nk * Hkv * d, torch.bfloat16),
            canary_view(B * Nk * Hkv * d, torch.bfloat16)]
    dq, dk, dv = (b[1].view(*shape) for b, shape in zip(bufs, ((B, Nq, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d))))
    attention_backward(q, k, v, o, lse, do, causal=True, window=window, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf, view, pad in bufs:
        assert not torch.isnan(view.float()).any()
        assert torch.all(buf[:pad] == 7) and torch.all(buf[pad + view.numel():] == 7)
    assert torch.all(wbuf[:4096] == 0x5A) and torch.all(wbuf[4096 + need:] == 0x5A)
    # causal with Nq > Nk: the first Nq - Nk rows see no key and get dQ = 0
    assert torch.all(dq[:, :Nq - Nk] == 0)


def test_backward_is_bitwise_deterministic_with_gqa_and_varlen():
    import torch
    q, k, v = qkv(1005, 2, 700, 700, 8, 2, 128, "f16")
    do = to_dev(synthetic.normal_bits(1005, synthetic.DO_ID, (2, 700, 8, 128), "f16"), "f16")
    o, lse = attention(q, k, v, causal=True)
    g1 = attention_backward(q, k, v, o, lse, do, causal=True)
    g2 = attention_backward(q, k, v, o, lse, do, causal=True)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    cu = torch.tensor([0, 300, 301, 700], dtype=torch.int32, device=device())
    qv, kv, vv, dov = (t[0] for t in (q, k, v, do))
    ov, lv = attention_varlen(qv, kv, vv, cu, cu, 399, causal=True)
    h1 = attention_varlen_backward(qv, kv, vv, ov, lv, dov, cu, cu, 399, 399, causal=True)
    h2 = attention_varlen_backward(qv, kv, vv, ov, lv, dov, cu, cu, 399, 399, causal=True)
    for a, b in zip(h1, h2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
