"""Seeded synthetic inputs for exact attention.

This module is the only code shared by the oracle and the HIP path. It holds
no attention arithmetic: it draws standard normals with numpy's PCG64 and
rounds them to the 16-bit storage formats (round to nearest, ties to even),
returning the raw 16-bit patterns. Both sides consume the same bits.

Recipe: one generator per (workload id, tensor id, batch index), so that any
batch slice can be regenerated on its own. Tensor ids: Q=0, K=1, V=2, and
dO=3 (the upstream gradient of a backward workload). Values
are N(0,1) in float32, multiplied by ``mult`` (an exact power of two in every
workload here), then rounded to fp16 or bf16.

Shapes follow the pages' [batch, seq_len, num_heads, head_dim] layout
("ampere_flash_attention_from_scratch" README, Performance Test table header;
"flash-attention-v100" README, How to use FlashAttention, flash_attn_func
arguments).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3
DTYPES = ("f16", "bf16")


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy rounds to nearest even) and return the bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with ties to even, at the bit level, for finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _slice_bits(workload_id, tensor_id, b, rest, dtype, mult):
    rng = np.random.default_rng([int(workload_id), int(tensor_id), int(b)])
    x = rng.standard_normal(rest, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return to_bits(x, dtype)


def normal_bits(workload_id: int, tensor_id: int, shape, dtype: str, mult: float = 1.0,
                batches=None, threads: int = 8) -> np.ndarray:
    """16-bit patterns of N(0,1)*mult, shape [B, N, H, d]; ``batches`` picks a subset of b.

    Each batch slice has its own generator, seeded [workload_id, tensor_id, b],
    so the result does not depend on ``batches`` or on the thread count.
    """
    B = int(shape[0])
    rest = tuple(int(s) for s in shape[1:])
    bs = list(range(B)) if batches is None else [int(b) for b in batches]
    out = np.empty((len(bs),) + rest, dtype=np.uint16)

    def fill(n):
        out[n] = _slice_bits(workload_id, tensor_id, bs[n], rest, dtype, mult)

    if threads > 1 and len(bs) > 1 and out.nbytes > (1 << 22):
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=min(threads, len(bs))) as ex:
            list(ex.map(fill, range(len(bs))))
    else:
        for n in range(len(bs)):
            fill(n)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask and input recipe."""
    name: str
    wid: int            # seed namespace
    B: int
    Nq: int
    Nk: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    causal: bool
    qk_mult: float = 1.0
    decode: bool = False
    num_splits: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def shapes(self):
        return ((self.B, self.Nq, self.Hq, self.d),
                (self.B, self.Nk, self.Hkv, self.d),
                (self.B, self.Nk, self.Hkv, self.d))

    def inputs(self, batches=None):
        """(q, k, v) as uint16 bit arrays, [B', N, H, d] for the chosen batch indices."""
        sq, sk, sv = self.shapes()
        q = normal_bits(self.wid, Q_ID, sq, self.dtype, self.qk_mult, batches)
        k = normal_bits(self.wid, K_ID, sk, self.dtype, self.qk_mult, batches)
        v = normal_bits(self.wid, V_ID, sv, self.dtype, 1.0, batches)
        return q, k, v

    def grad_out(self, batches=None):
        """dO as uint16 bits shaped like q (backward workloads)."""
        return normal_bits(self.wid, DO_ID, self.shapes()[0], self.dtype, 1.0, batches)

    def pairs(self) -> int:
        """Number of unmasked (query, key) pairs per (b, head)."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return sum(max(0, min(self.Nk, i + off + 1)) for i in range(self.Nq))

    def flops(self) -> float:
        """Forward FLOPs counting both products over unmasked pairs: 4 * B * Hq * pairs * d."""
        return 4.0 * self.B * self.Hq * self.pairs() * self.d


def _build():
    w = []
    w.append(Workload("tiny_f16_128", 0, 1, 128, 128, 2, 2, 64, "f16", False))
    w.append(Workload("headline_f16_1024", 1, 16, 1024, 1024, 32, 32, 128, "f16", False))
    wid = 2
    for n in (2048, 4096, 8192):
        for causal in (False, True):
            w.append(Workload(f"long_f16_{n}_{'causal' if causal else 'full'}", wid, 16, n, n, 32, 32,
                              128, "f16", causal))
            wid += 1
    for causal in (False, True):
        w.append(Workload(f"long_bf16_8192_sharp_{'causal' if causal else 'full'}", wid, 16, 8192, 8192,
                          32, 32, 128, "bf16", causal, qk_mult=2.0))
        wid += 1
    for d in (32, 64, 96, 128, 192, 256):
        w.append(Workload(f"gqa_bf16_2048_d{d}", wid, 8, 2048, 2048, 32, 8, d, "bf16", True))
        wid += 1
    for nq in (1, 8):
        w.append(Workload(f"decode_bf16_nq{nq}", wid, 8, nq, 8192, 32, 8, 128, "bf16", False,
                          decode=True, num_splits=16))
        wid += 1
    # backward: the pages' fwd+bwd benchmark setting at N = 4096 (hidden 2048 as
    # 16 heads of 128, batch 16K / N = 4)
    for causal in (False, True):
        w.append(Workload(f"bwd_bf16_4096_{'causal' if causal else 'full'}", wid, 4, 4096, 4096, 16, 16,
                          128, "bf16", causal))
        wid += 1
    return {x.name: x for x in w}


WORKLOADS = _build()


def block_table(workload_id: int, B: int, max_pages: int, num_pages: int) -> np.ndarray:
    """int32 [B, max_pages] page indices for a paged KV cache: a seeded permutation
    of the pool's pages, so that no page is shared and logical order is scrambled."""
    if num_pages < B * max_pages:
        raise ValueError("the pool needs at least B * max_pages pages")
    rng = np.random.default_rng([int(workload_id), 7])
    return rng.permutation(num_pages)[: B * max_pages].astype(np.int32).reshape(B, max_pages)
