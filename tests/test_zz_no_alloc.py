"""GPU check of fa_decode_splitkv_noalloc, the decode entry point that allocates
nothing (its partials live in the library's fixed device scratch), through the
C ABI: two calls in a row, the second on a smaller problem, each equal bit for
bit to fa_decode_splitkv (the same kernels with a caller's workspace) on the
same inputs and within the parity bounds of the fp64 oracle."""
import math

import pytest

import _compare as cmp
import oracle
import synthetic
from gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu

from exact_tiled_attention_21_amd import decode, decode_noalloc  # noqa: E402

# (workload id, B, Nq, Nk, Hq, Hkv, d, dtype, splits, causal): the decode workload
# with Nq = 8 (16 MiB of partials), then a smaller, ragged, causal problem
CALLS = [(1200, 8, 8, 8192, 32, 8, 128, "bf16", 16, False),
         (1201, 2, 3, 1000, 8, 2, 64, "f16", 7, True)]


def test_noalloc_matches_workspace_entry_point():
    import torch
    for wid, B, Nq, Nk, Hq, Hkv, d, dtype, S, causal in CALLS:
        print(f"[noalloc] wid={wid} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} {dtype} S={S} causal={causal}",
              flush=True)
        qb = synthetic.normal_bits(wid, 0, (B, Nq, Hq, d), dtype)
        kb = synthetic.normal_bits(wid, 1, (B, Nk, Hkv, d), dtype)
        vb = synthetic.normal_bits(wid, 2, (B, Nk, Hkv, d), dtype)
        q, k, v = (to_dev(x, dtype) for x in (qb, kb, vb))
        scale = 1.0 / math.sqrt(d)
        o_ws, l_ws = decode(q, k, v, num_splits=S, causal=causal, scale=scale)
        o_na = torch.full_like(o_ws, float("nan"))
        l_na = torch.full_like(l_ws, float("nan"))
        decode_noalloc(q, k, v, num_splits=S, causal=causal, scale=scale, out=o_na, lse=l_na)
        torch.cuda.synchronize()
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32))
        o_ref, l_ref = oracle.attention_bits(qb, kb, vb, dtype, causal=causal, scale=scale)
        what = f"noalloc wid={wid}"
        cmp.check_o(to_np(o_na), o_ref, dtype, what)
        cmp.check_lse(to_np(l_na), l_ref, what)
