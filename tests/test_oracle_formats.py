"""Pins for the oracle's number formats against numpy / torch conversions."""
import numpy as np
import pytest
import torch

import oracle as O


def test_f16_decode_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = O.f16_decode(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero preserved
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _samples(rng, n=200000):
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(1e6), n))
    x = mags * rng.choice([-1.0, 1.0], n)
    # exact midpoints between neighbouring fp16 values (ties), incl. subnormal and top binade
    h = rng.integers(0, 0x7BFF, 20000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    mid = mid * rng.choice([-1.0, 1.0], mid.size)
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9, 2.0**-24, 2.0**-25,
                        2.0**-25 * 1.0000001, 2.0**-14, 2.0**-14 * (1 - 2**-12), 1.0 + 2**-11, 1.0 + 3 * 2**-11])
    return np.concatenate([x, mid, lo, special, -special])


def test_f16_encode_rne_matches_numpy():
    rng = np.random.default_rng(1)
    x = _samples(rng)
    ref = x.astype(np.float16).view(np.uint16)
    got = O.f16_encode(x, O.RNE)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("mode", [O.RD, O.RU])
def test_f16_encode_directed(mode):
    rng = np.random.default_rng(2)
    x = _samples(rng)
    x = x[np.abs(x) <= 65504.0]
    got = O.f16_encode(x, mode).view(np.float16).astype(np.float64)
    near = x.astype(np.float16)
    cand = np.stack([np.nextafter(near, np.float16(-np.inf)), near,
                     np.nextafter(near, np.float16(np.inf))]).astype(np.float64)
    if mode == O.RD:   # largest fp16 <= x
        ok = np.where(cand <= x, cand, -np.inf).max(axis=0)
    else:              # smallest fp16 >= x
        ok = np.where(cand >= x, cand, np.inf).min(axis=0)
    assert np.array_equal(got, ok)
    # overflow handling: toward zero saturates, away from zero gives infinity
    big = np.array([70000.0, -70000.0])
    g = O.f16_encode(big, mode).view(np.float16).astype(np.float64)
    if mode == O.RD:
        assert g[0] == 65504.0 and g[1] == -np.inf
    else:
        assert g[0] == np.inf and g[1] == -65504.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    h = rng.integers(0, 65536, 100000).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]           # drop inf/nan patterns
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_decode(h), ref)
