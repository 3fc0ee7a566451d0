"""The Python binding refuses caller-supplied buffers the kernels could not write
into safely (wrong shape, dtype, device or layout) before any library call, and
a correct caller-supplied buffer gives the same bits as the allocating path."""
import pytest

pytestmark = pytest.mark.gpu

import torch  # noqa: E402

from exact_tiled_attention_21_amd import (attention, attention_backward, attention_varlen, decode,  # noqa: E402
                                          decode_workspace_bytes)


@pytest.fixture(scope="module")
def qkv():
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    q, k, v = (torch.randn((2, 70, 4, 64), generator=g, device="cuda").half() for _ in range(3))
    return q, k, v


def test_forward_output_buffers(qkv):
    q, k, v = qkv
    o, lse = attention(q, k, v, causal=True)
    out, lse_out = torch.empty_like(q), torch.empty_like(lse)
    o2, lse2 = attention(q, k, v, causal=True, out=out, lse=lse_out)
    assert o2.data_ptr() == out.data_ptr() and lse2.data_ptr() == lse_out.data_ptr()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    bad_out = [torch.empty((2, 69, 4, 64), dtype=q.dtype, device="cuda"),      # too small
               torch.empty_like(q, dtype=torch.bfloat16),                      # other dtype
               torch.empty_like(q, device="cpu"),                              # host memory
               torch.empty((2, 4, 70, 64), dtype=q.dtype, device="cuda").transpose(1, 2)]   # strided
    for b in bad_out:
        with pytest.raises(ValueError):
            attention(q, k, v, out=b)
    for b in (torch.empty((2, 4, 69), device="cuda"), torch.empty_like(lse, dtype=torch.float16),
              torch.empty_like(lse, device="cpu")):
        with pytest.raises(ValueError):
            attention(q, k, v, lse=b)


def test_decode_workspace_and_outputs(qkv):
    q, k, v = qkv
    qd = q[:, :1].contiguous()
    o, lse = decode(qd, k, v, num_splits=4)
    ws = torch.empty(decode_workspace_bytes(2, 1, 4, 64, 4), dtype=torch.uint8, device="cuda")
    o2, lse2 = decode(qd, k, v, num_splits=4, workspace=ws)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    with pytest.raises(ValueError):
        decode(qd, k, v, num_splits=4, workspace=ws.cpu())
    with pytest.raises(ValueError):
        decode(qd, k, v, num_splits=4, out=torch.empty_like(q))


def test_backward_gradient_buffers(qkv):
    q, k, v = qkv
    o, lse = attention(q, k, v)
    do = torch.randn_like(q)
    dq, dk, dv = attention_backward(q, k, v, o, lse, do)
    given = [torch.empty_like(x) for x in (q, k, v)]
    dq2, dk2, dv2 = attention_backward(q, k, v, o, lse, do, dq=given[0], dk=given[1], dv=given[2])
    assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), (dq2, dk2, dv2)))
    with pytest.raises(ValueError):
        attention_backward(q, k, v, o, lse, do, dk=torch.empty((2, 69, 4, 64), dtype=q.dtype, device="cuda"))
    with pytest.raises(ValueError):
        attention_backward(q, k, v, o, lse, do, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        attention_backward(q, k, v, o.cpu(), lse, do)


def test_varlen_index_tensors_on_the_device(qkv):
    q, k, v = qkv
    qp, kp, vp = (x.reshape(140, 4, 64) for x in (q, k, v))
    cu = torch.tensor([0, 70, 140], dtype=torch.int32)
    with pytest.raises(ValueError):
        attention_varlen(qp, kp, vp, cu, cu.cuda(), 70)
    o, _ = attention_varlen(qp, kp, vp, cu.cuda(), cu.cuda(), 70)
    assert torch.equal(o.reshape(q.shape), attention(q, k, v)[0])


def test_varlen_max_seqlen_below_a_sequence_is_refused(qkv):
    """max_seqlen_q / max_seqlen_k sizes the grid and the workspace; one below some
    sequence's length would leave rows unwritten (forward) or clip that sequence
    (backward), so the binding checks it against the prefix sums."""
    from exact_tiled_attention_21_amd import attention_varlen_backward
    q, k, v = qkv
    qp, kp, vp = (x.reshape(140, 4, 64) for x in (q, k, v))
    cu = torch.tensor([0, 30, 140], dtype=torch.int32, device="cuda")   # lengths 30 and 110
    with pytest.raises(ValueError, match="max_seqlen_q"):
        attention_varlen(qp, kp, vp, cu, cu, 100)
    o, lse = attention_varlen(qp, kp, vp, cu, cu, 110)
    do = torch.ones_like(qp)
    with pytest.raises(ValueError, match="max_seqlen_q"):
        attention_varlen_backward(qp, kp, vp, o, lse, do, cu, cu, 100, 110)
    with pytest.raises(ValueError, match="max_seqlen_k"):
        attention_varlen_backward(qp, kp, vp, o, lse, do, cu, cu, 110, 100)
    attention_varlen_backward(qp, kp, vp, o, lse, do, cu, cu, 110, 110)
