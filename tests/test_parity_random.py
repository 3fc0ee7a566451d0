"""GPU parity against the fp64 oracle on seeded random configurations.

The other parity files pick their shapes by hand (tile edges, ragged tails,
every head dim, fully masked rows). This one draws the shape, head grouping,
head dim, dtype, mask, scale, for decode the split count and paging, and for
packed batches the number of sequences and their query and key lengths (empty
ones included) from a fixed seed, so that combinations nobody listed are
covered too; a few long single sequences (2048 to 4800 rows) reach the wide
forward shape. Sizes stay small enough for the oracle to finish in about a
second per case.
"""
import math
import os

import numpy as np
import pytest

import test_parity_bwd as bwd
import test_parity_bwd_varlen as bvl
import test_parity_decode as dec
import test_parity_decode_paged as paged
import test_parity_fwd as fwd
import test_parity_fwd_varlen as fvl
import test_parity_fwd_window as win

pytestmark = pytest.mark.gpu

HEAD_DIMS = (32, 64, 96, 128, 192, 256)
# FA_RANDOM_SEED and FA_RANDOM_SCALE (a multiplier of the case counts) widen the
# sweep for a longer run; the defaults are the suite's fixed configurations
_rng = np.random.default_rng(int(os.environ.get("FA_RANDOM_SEED", "20261203")))
_SCALE = float(os.environ.get("FA_RANDOM_SCALE", "1"))


def _heads():
    hkv = int(_rng.choice([1, 2, 4]))
    return hkv * int(_rng.choice([1, 2, 3, 4])), hkv


def _scale(d):
    # the default most of the time; otherwise a random magnitude and sign
    if _rng.random() < 0.6:
        return None
    return float(_rng.choice([-1.0, 1.0]) * _rng.uniform(0.3, 2.0) / math.sqrt(d))


def _mask(nq, nk):
    r = _rng.random()
    if r < 0.4:
        return False, (-1, -1)
    if r < 0.7:
        return True, (-1, -1)
    wl = int(_rng.choice([-1, int(_rng.integers(0, nk + 1))]))
    wr = int(_rng.choice([-1, int(_rng.integers(0, nk + 1))]))
    return False, (wl, wr)


def _fwd_cases(n):
    out = []
    for i in range(n):
        hq, hkv = _heads()
        nq, nk = int(_rng.integers(1, 400)), int(_rng.integers(1, 400))
        d = int(_rng.choice(HEAD_DIMS))
        causal, window = _mask(nq, nk)
        out.append((6000 + i, int(_rng.integers(1, 4)), nq, nk, hq, hkv, d, str(_rng.choice(["f16", "bf16"])),
                    causal, window, _scale(d)))
    return out


def _bwd_cases(n):
    out = []
    for i in range(n):
        hq, hkv = _heads()
        nq, nk = int(_rng.integers(1, 300)), int(_rng.integers(1, 300))
        d = int(_rng.choice(HEAD_DIMS))
        causal, window = _mask(nq, nk)
        out.append((6100 + i, int(_rng.integers(1, 3)), nq, nk, hq, hkv, d, str(_rng.choice(["f16", "bf16"])),
                    causal, window, _scale(d)))
    return out


def _dec_cases(n):
    out = []
    for i in range(n):
        hq, hkv = _heads()
        d = int(_rng.choice(HEAD_DIMS))
        nq = int(_rng.integers(1, 9))
        page = int(_rng.choice([0, 32, 64, 256]))          # 0: contiguous cache
        out.append((6200 + i, int(_rng.integers(1, 6)), nq, int(_rng.integers(1, 3000)), hq, hkv, d,
                    str(_rng.choice(["f16", "bf16"])), int(_rng.integers(1, 65)), bool(_rng.random() < 0.3),
                    page, _scale(d)))
    return out


def _varlen_cases(n, base, maxlen):
    out = []
    for i in range(n):
        hq, hkv = _heads()
        nseq = int(_rng.integers(1, 7))
        lq = [int(x) for x in _rng.integers(0, maxlen + 1, size=nseq)]
        # self-attention lengths most of the time, otherwise independent key lengths
        lk = list(lq) if _rng.random() < 0.5 else [int(x) for x in _rng.integers(0, maxlen + 1, size=nseq)]
        if sum(lq) == 0:
            lq[0] = 1
        if sum(lk) == 0:
            lk[0] = 1
        out.append((base + i, tuple(lq), tuple(lk), hq, hkv, int(_rng.choice(HEAD_DIMS)),
                    str(_rng.choice(["f16", "bf16"])), bool(_rng.random() < 0.5)))
    return out


def _n(k):
    return max(1, int(round(k * _SCALE)))


FWD = _fwd_cases(_n(80))
BWD = _bwd_cases(_n(48))
DEC = _dec_cases(_n(48))
FVL = _varlen_cases(_n(24), 6300, 300)
BVL = _varlen_cases(_n(16), 6400, 200)


def _long_cases(n):
    # long single sequences (the 256-row workgroups of fp16 d = 128 without a
    # band start at 3072 query rows), a few heads so the oracle stays quick
    out = []
    for i in range(n):
        hkv = int(_rng.choice([1, 2]))
        hq = hkv * int(_rng.choice([1, 2]))
        nq, nk = int(_rng.integers(2048, 4800)), int(_rng.integers(1, 4800))
        d = int(_rng.choice([64, 128, 128]))
        dtype = str(_rng.choice(["f16", "f16", "bf16"]))
        causal, window = _mask(nq, nk)
        out.append((6500 + i, 1, nq, nk, hq, hkv, d, dtype, causal, window, _scale(d)))
    return out


LONG = _long_cases(_n(6))


def _id(c):
    return "-".join(str(x) for x in c[1:])


@pytest.mark.parametrize("case", FWD, ids=_id)
def test_forward(case):
    wid, B, nq, nk, hq, hkv, d, dtype, causal, window, scale = case
    if window == (-1, -1):
        fwd.run_full(wid, B, nq, nk, hq, hkv, d, dtype, causal, scale=scale)
    else:
        win.run(wid, B, nq, nk, hq, hkv, d, dtype, window)


@pytest.mark.parametrize("case", BWD, ids=_id)
def test_backward(case):
    wid, B, nq, nk, hq, hkv, d, dtype, causal, window, scale = case
    bwd.run_full(wid, B, nq, nk, hq, hkv, d, dtype, causal, scale=scale, window=window)


@pytest.mark.parametrize("case", DEC, ids=_id)
def test_decode(case):
    wid, B, nq, nk, hq, hkv, d, dtype, splits, causal, page, scale = case
    if page == 0:
        dec.run(wid, B, nq, nk, hq, hkv, d, dtype, splits, causal=causal, scale=scale)
    else:
        max_pages = (nk + page - 1) // page
        lens = [int(x) for x in _lens(wid, B, max_pages * page)]
        paged.run(wid, B, nq, hq, hkv, d, dtype, page, max_pages, lens, splits=splits, causal=causal, scale=scale)


def _lens(wid, B, cap):
    r = np.random.default_rng(wid)
    return r.integers(0, cap + 1, size=B)


def _vid(c):
    return f"{len(c[1])}seq-{c[3]}-{c[4]}-{c[5]}-{c[6]}-{'causal' if c[7] else 'full'}-{c[0]}"


@pytest.mark.parametrize("case", FVL, ids=_vid)
def test_forward_varlen(case):
    wid, lq, lk, hq, hkv, d, dtype, causal = case
    fvl.run(wid, lq, lk, hq, hkv, d, dtype, causal=causal)


@pytest.mark.parametrize("case", BVL, ids=_vid)
def test_backward_varlen(case):
    wid, lq, lk, hq, hkv, d, dtype, causal = case
    bvl.run(wid, lq, lk, hq, hkv, d, dtype, causal=causal)


@pytest.mark.parametrize("case", LONG, ids=_id)
def test_forward_long(case):
    test_forward(case)
