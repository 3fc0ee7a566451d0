"""GPU parity at the widest rows the C ABI accepts: Hq * d = 2^22 elements.

65536 heads of 64 (one KV head per query head), so one [.., H, d] row spans
8 MiB and a 64-key tile spans about half a GiB of the 32-bit byte offsets the
kernels address a tile with; 100 keys and queries leave the second key tile
ragged and the query tile part empty. The forward (no mask and causal), the
backward (on the forward's own O and LSE) and the split-KV decode (the same
bits viewed as 32768 heads of 128) run over the whole problem on the GPU; the
oracle checks a sample of heads at the start, the middle and the end of the
rows (heads are independent when every query head has its own KV head).
"""
import math

import numpy as np
import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import attention, attention_backward, decode  # noqa: E402

WID, N, H, D, DTYPE = 990, 100, 65536, 64, "f16"


def sample_heads(h):
    rng = np.random.default_rng([WID, h])
    fixed = [0, 1, 63, 64, 4095, 4096, h // 2 - 1, h // 2, h - 65, h - 2, h - 1]
    return sorted(set(fixed) | set(int(x) for x in rng.choice(h, 5, replace=False)))


@pytest.fixture(scope="module")
def bits():
    shape = (1, N, H, D)
    print(f"[limits] drawing 4 x {shape} {DTYPE}", flush=True)
    return tuple(synthetic.normal_bits(WID, t, shape, DTYPE)
                 for t in (synthetic.Q_ID, synthetic.K_ID, synthetic.V_ID, synthetic.DO_ID))


@pytest.fixture(scope="module")
def dev(bits):
    return tuple(to_dev(b, DTYPE) for b in bits)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_at_the_widest_rows(bits, dev, causal):
    qb, kb, vb, dob = bits
    qd, kd, vd, dod = dev
    scale = 1.0 / math.sqrt(D)
    what = f"B=1 N={N} H={H} d={D} {DTYPE} causal={causal}"
    print(f"[limits] forward + backward {what}", flush=True)
    o, lse = attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    hs = sample_heads(H)
    q, k, v, do = (oracle.widen(x[:, :, hs], DTYPE) for x in (qb, kb, vb, dob))
    o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, scale=scale)
    cmp.check_o(to_np(o[:, :, hs]), o_ref, DTYPE, what)
    cmp.check_lse(to_np(lse[:, hs]), lse_ref, what)
    ref = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    mag = oracle.backward_magnitudes(q, k, v, do, causal=causal, scale=scale)
    flo = oracle.backward_operand_sums(q, k, do, causal=causal, scale=scale)
    for g, r, m, f, n in zip((dq, dk, dv), ref, mag, flo, ("dq", "dk", "dv")):
        cmp.check_grad(to_np(g[:, :, hs]), r, m, DTYPE, f"{what} {n}", floor=f)


def test_decode_at_the_widest_rows(bits, dev):
    """The forward's bits reinterpreted: K and V as a cache of 100 keys of 32768
    heads of 128, query row 0 as one decode step of 32768 heads."""
    qb, kb, vb, _ = bits
    qd, kd, vd, _ = dev
    h2, d2 = H // 2, 2 * D
    qb2, kb2, vb2 = qb[:, :1].reshape(1, 1, h2, d2), kb.reshape(1, N, h2, d2), vb.reshape(1, N, h2, d2)
    scale = 1.0 / math.sqrt(d2)
    what = f"decode B=1 Nq=1 Nk={N} H={h2} d={d2} {DTYPE} S=4"
    print(f"[limits] {what}", flush=True)
    o, lse = decode(qd[:, :1].reshape(1, 1, h2, d2), kd.view(1, N, h2, d2), vd.view(1, N, h2, d2),
                    num_splits=4, scale=scale)
    hs = sample_heads(h2)
    o_ref, lse_ref = oracle.attention_bits(qb2[:, :, hs], kb2[:, :, hs], vb2[:, :, hs], DTYPE, scale=scale)
    cmp.check_o(to_np(o[:, :, hs]), o_ref, DTYPE, what)
    cmp.check_lse(to_np(lse[:, hs]), lse_ref, what)


# Tensors larger than 4 GiB: every byte offset past the first 4 GiB would wrap in
# 32 bits. The batches in between only have to hold N(0,1) values, so they are
# drawn on the device (torch's seeded generator); the first and the last batch
# hold the shared host recipe's bits and are checked whole against the oracle.
BIG_WID = 991


def big_tensor(tensor_id, shape, dtype, edge_bits):
    import torch
    from gpu_util import device
    dev = device()
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(BIG_WID * 16 + tensor_id)
    x = torch.empty(shape, dtype=tdt, device=dev)
    for b0 in range(0, shape[0], 64):
        n = min(64, shape[0] - b0)
        x[b0:b0 + n] = torch.randn((n,) + tuple(shape[1:]), generator=g, device=dev, dtype=torch.float32).to(tdt)
    x[0:1] = to_dev(edge_bits[0:1], dtype)
    x[-1:] = to_dev(edge_bits[1:2], dtype)
    torch.cuda.synchronize()
    return x


def big_inputs(shapes, dtype, ids):
    edges = [synthetic.normal_bits(BIG_WID, t, s, dtype, batches=[0, s[0] - 1]) for t, s in zip(ids, shapes)]
    return edges, [big_tensor(t, s, dtype, e) for t, s, e in zip(ids, shapes, edges)]


def test_forward_and_backward_beyond_4_gib():
    """B = 600, 1024 tokens, 32 heads of 128, bf16: 4.7 GiB per tensor."""
    import torch
    B, N, H, d, dtype = 600, 1024, 32, 128, "bf16"
    shape = (B, N, H, d)
    print(f"[limits] forward + backward {shape} {dtype}", flush=True)
    edges, (q, k, v, do) = big_inputs([shape] * 4, dtype,
                                      [synthetic.Q_ID, synthetic.K_ID, synthetic.V_ID, synthetic.DO_ID])
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, lse = attention(q, k, v, causal=causal, scale=scale)
        grads = attention_backward(q, k, v, o, lse, do, causal=causal, scale=scale) if causal else None
        for n, b in enumerate((0, B - 1)):
            what = f"{shape} {dtype} causal={causal} b={b}"
            qb, kb, vb, dob = (oracle.widen(e[n:n + 1], dtype) for e in edges)
            o_ref, lse_ref = oracle.attention(qb, kb, vb, causal=causal, scale=scale)
            cmp.check_o(to_np(o[b:b + 1]), o_ref, dtype, what)
            cmp.check_lse(to_np(lse[b:b + 1]), lse_ref, what)
            if grads is not None:
                ref = oracle.backward(qb, kb, vb, dob, causal=True, scale=scale)
                mag = oracle.backward_magnitudes(qb, kb, vb, dob, causal=True, scale=scale)
                flo = oracle.backward_operand_sums(qb, kb, dob, causal=True, scale=scale)
                for g, r, m, f, name in zip(grads, ref, mag, flo, ("dq", "dk", "dv")):
                    cmp.check_grad(to_np(g[b:b + 1]), r, m, dtype, f"{what} {name}", floor=f)
        del o, lse, grads
    del q, k, v, do
    torch.cuda.empty_cache()


def test_decode_beyond_4_gib():
    """A cache of 64 sequences of 8300 keys, 32 KV heads of 128, bf16 (4.3 GB per
    tensor); 128 query heads (groups of 4), one query row each."""
    import torch
    B, Nk, Hq, Hkv, d, dtype = 64, 8300, 128, 32, 128, "bf16"
    print(f"[limits] decode B={B} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype}", flush=True)
    edges, (q, k, v) = big_inputs([(B, 1, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d)], dtype,
                                  [synthetic.Q_ID, synthetic.K_ID, synthetic.V_ID])
    scale = 1.0 / math.sqrt(d)
    o, lse = decode(q, k, v, num_splits=16, scale=scale)
    for n, b in enumerate((0, B - 1)):
        what = f"decode B={B} Nk={Nk} Hq={Hq} Hkv={Hkv} b={b}"
        o_ref, lse_ref = oracle.attention_bits(edges[0][n:n + 1], edges[1][n:n + 1], edges[2][n:n + 1], dtype,
                                               scale=scale)
        cmp.check_o(to_np(o[b:b + 1]), o_ref, dtype, what)
        cmp.check_lse(to_np(lse[b:b + 1]), lse_ref, what)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
