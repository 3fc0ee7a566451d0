"""Helpers for the GPU parity tests: device upload of the shared 16-bit inputs
and oracle references (whole tensors, or sampled rows at large sizes)."""
from __future__ import annotations

import numpy as np

import oracle


def device():
    import torch
    assert torch.cuda.is_available(), "GPU test needs a ROCm device"
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device())
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def oracle_rows(qb, kb, vb, dtype, rows, causal, scale):
    """Oracle O [1, len(rows), Hq, d] and LSE [1, Hq, len(rows)] for query rows `rows` of
    one batch element (bit arrays [1, N, H, d]). For causal rows it uses the pinned
    prefix identity: causal row i equals non-causal attention over keys 0..i+Nk-Nq."""
    q = oracle.widen(qb, dtype)
    k = oracle.widen(kb, dtype)
    v = oracle.widen(vb, dtype)
    nq, nk = q.shape[1], k.shape[1]
    rows = list(rows)
    if not causal:
        return oracle.attention(q[:, rows], k, v, scale=scale)
    hq, d = q.shape[2], q.shape[3]
    o = np.zeros((1, len(rows), hq, d))
    lse = np.full((1, hq, len(rows)), -np.inf)
    for n, i in enumerate(rows):
        end = min(nk, i + nk - nq + 1)
        if end <= 0:
            continue
        oi, li = oracle.attention(q[:, i:i + 1], k[:, :end], v[:, :end], scale=scale)
        o[:, n] = oi[:, 0]
        lse[:, :, n] = li[:, :, 0]
    return o, lse
