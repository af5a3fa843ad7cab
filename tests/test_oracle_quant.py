"""Pins for the group-wise affine quantizer (paper §2.1) and the packed layout."""
import numpy as np
import pytest

import oracle as O


def _groups(rng, n, g):
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            v = rng.normal(size=g)
        elif kind == 1:
            v = rng.normal(size=g) * np.exp(rng.normal())
            v[rng.integers(g)] *= 8.0                       # an outlier
        elif kind == 2:
            v = rng.normal(size=g) + 50.0                   # offset far from zero
        elif kind == 3:
            v = -np.abs(rng.normal(size=g)) * 1e-3          # tiny negative values
        else:
            v = rng.uniform(-3, 3, size=g)
        out.append(v)
    return out


def _f16(h):
    return float(np.uint16(h).view(np.float16))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantizer_invariants(bits):
    rng = np.random.default_rng(bits)
    qmax = 2 ** bits - 1
    near_constant = 0
    for v in _groups(rng, 600, 32):
        o16, s16, codes, delta, pre_o, pre_s = O.group_quant(v, bits)
        o, s = _f16(o16), _f16(s16)
        mn, mx = v.min(), v.max()
        # o is the largest fp16 <= min; s the smallest fp16 >= (max - o)/qmax
        assert o <= mn < float(np.nextafter(np.float16(o), np.float16(np.inf)))
        assert s >= (mx - o) / qmax > float(np.nextafter(np.float16(s), np.float16(-np.inf)))
        assert pre_o == mn and abs(pre_s - (mx - o) / qmax) <= 1e-15 * abs(pre_s)
        assert codes.max() <= qmax
        deq = o + s * codes.astype(np.float64)
        # no clipping: every element within half a step (textbook uniform quantizer)
        assert np.all(np.abs(v - deq) <= s / 2 * (1 + 2 ** -20))
        # brute force: the code is the nearest level (exact ties excluded by delta)
        levels = o + s * np.arange(qmax + 1)
        best = np.abs(v[:, None] - levels[None, :]).argmin(axis=1)
        tie = delta < 1e-9
        assert np.array_equal(codes[~tie], best[~tie])
        # the max maps to the top level; the min to level 0 unless the group is near-constant
        # (with a normal fp16 s, rounding s up costs at most a factor 1 + 2^-10, so
        # (max - o)/s >= qmax/(1 + 2^-10) > qmax - 1/2 for qmax < 512)
        if s >= 2.0 ** -14:
            assert codes[v.argmax()] == qmax
        if codes[v.argmin()] != 0:
            # only possible when the rounding of o (< one fp16 spacing of min) reaches half
            # a step: max - min <= 2 qmax (min - o) < 2 qmax spacing(min)
            near_constant += 1
            spacing = max(2.0 ** -10 * abs(mn), 2.0 ** -24)
            assert (mx - mn) <= 2 * qmax * spacing
    if bits <= 4:
        assert near_constant <= 3


def test_int2_uses_all_four_levels():
    v = np.linspace(-1.0, 2.0, 32)
    o16, s16, codes, *_ = O.group_quant(v, 2)
    assert set(codes.tolist()) == {0, 1, 2, 3}            # affine: four distinct levels
    # a zero-centred symmetric grid would only offer three for this group (paper §2.1)
    assert _f16(o16) <= -1.0 and _f16(o16) + 3 * _f16(s16) >= 2.0


def test_constant_group():
    for val in [0.0, 1.5, -2.25, 0.1]:
        v = np.full(32, val)
        o16, s16, codes, *_ = O.group_quant(v, 2)
        o = _f16(o16)
        assert np.all(codes == 0) or _f16(s16) > 0
        if float(np.float16(val)) == val:                      # exactly representable -> s = 0, lossless
            assert _f16(s16) == 0.0 and np.all(codes == 0) and o == val
        deq = o + _f16(s16) * codes
        assert np.all(np.abs(deq - v) <= abs(val) * 2 ** -10 + 1e-30)


@pytest.mark.parametrize("bits,g", [(2, 32), (4, 32), (8, 32), (16, 32), (2, 16), (4, 16), (2, 64)])
def test_pack_roundtrip(bits, g):
    rng = np.random.default_rng(bits * 100 + g)
    for _ in range(50):
        c = rng.integers(0, 2 ** bits, g).astype(np.uint16)
        b = O.pack_group(c, bits)
        assert b.size == g * bits // 8
        assert np.array_equal(O.unpack_group(b, g, bits), c)


@pytest.mark.parametrize("bits,g", [(2, 32), (4, 32), (8, 32), (16, 32), (2, 16), (4, 16)])
def test_pack_layout_single_bit_probe(bits, g):
    """Each element's least significant code bit lands where the layout rule says.

    Rule: element e sits in half h = e // (g/2), index k = e % (g/2); half-word
    j = k // (16/bits) of that half; bit offset bits*(k % (16/bits)); word j is
    (half-word j of half 0) | (half-word j of half 1) << 16, little-endian.
    """
    half, per = g // 2, 16 // bits
    for e in range(g):
        c = np.zeros(g, np.uint16)
        c[e] = 1
        b = O.pack_group(c, bits)
        bitpos = np.nonzero(np.unpackbits(b, bitorder="little"))[0]
        h, k = divmod(e, half)
        j, p = divmod(k, per)
        expect = 32 * j + 16 * h + bits * p
        assert bitpos.tolist() == [expect], (e, bitpos, expect)


def _f16_up(x):
    """Smallest float16 >= x (numpy's conversion rounds to nearest; step up if below)."""
    h = np.float16(x)
    if float(h) < x:
        h = np.nextafter(h, np.float16(np.inf))
    return h


def test_offset_beyond_fp16_range_saturates():
    """A group whose minimum is below -65504 keeps the most negative finite fp16
    offset; values below it clip to code 0 and the rest follow the usual rule."""
    v = np.linspace(-70000.0, 1000.0, 32)
    for bits in (2, 4):
        qmax = 2 ** bits - 1
        o16, s16, codes, _, pre_o, pre_s = O.group_quant(v, bits)
        assert np.isneginf(np.float16(v.min()))              # plain fp16 rounding would overflow
        assert o16 == int(np.float16(-65504.0).view(np.uint16))
        s = _f16(s16)
        assert s == float(_f16_up((v.max() + 65504.0) / qmax))
        assert pre_s == (v.max() + 65504.0) / qmax
        levels = -65504.0 + s * np.arange(qmax + 1)
        best = np.abs(v[:, None] - levels[None, :]).argmin(axis=1)   # nearest level, clipping included
        assert np.array_equal(codes, best)
        assert codes[0] == 0 and codes[-1] == qmax


def test_scale_beyond_fp16_range_saturates():
    """(max - o)/(2^b - 1) above 65504 keeps the largest finite fp16 scale; values past
    o + (2^b - 1) * 65504 clip to the top code."""
    v = np.concatenate([[0.0, 250000.0], np.linspace(1.0, 240000.0, 30)])
    o16, s16, codes, _, pre_o, pre_s = O.group_quant(v, 2)
    assert _f16(o16) == 0.0 and pre_s == 250000.0 / 3
    assert np.isinf(np.float16(pre_s))
    assert s16 == int(np.float16(65504.0).view(np.uint16))
    expect = np.clip(np.round(v / 65504.0), 0, 3)            # no exact ties in these values
    assert np.array_equal(codes, expect.astype(np.uint16))
    assert codes[1] == 3 and codes[0] == 0
