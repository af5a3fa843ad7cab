"""Oracle pins for anchor loop groups (paper §5 "Models": loops partitioned into
independent groups, each with its own anchor) and the First-loop policy (§3.2).
Each pin compares the oracle with itself on a differently arranged problem whose
answer the paper's definitions fix: independent groups, a one-loop group, and
the mirror image between First-loop and Last-loop."""
import numpy as np
import pytest

import oracle as O

D, T = 64, 40
LAST, PREV, FIRST = O.LAST_LOOP, O.PREV_LOOP, O.FIRST_LOOP


def _inputs(L, seed=0):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((T, D))
    X = np.stack([(0.7 + 0.05 * r) * base + (0.3 / (r + 1)) * rng.standard_normal((T, D)) for r in range(L)])
    bf = (X.astype(np.float32).view(np.uint32) + 0x8000 >> 16).astype(np.uint16)   # to bf16 bits (RNE-ish)
    H = O.rotation(D, D, rng.choice([-1, 1], D)).astype(np.float32)
    return bf, H


def _series(X, H, bits, policy, loop_group=0):
    cfg = O.Config(D=D, bits=list(bits), policy=policy, loop_group=loop_group)
    return cfg, O.quantize_series(cfg, X, H, diagnostics=False)


def _same(a: O.Series, ra: int, b: O.Series, rb: int):
    assert np.array_equal(a.codes[ra], b.codes[rb])
    assert np.array_equal(a.meta[ra], b.meta[rb])


@pytest.mark.parametrize("policy", [LAST, PREV, FIRST])
def test_groups_are_independent(policy):
    """Eight loops in two groups of four = two separate four-loop series."""
    X, H = _inputs(8)
    bits = [2, 2, 4, 4, 4, 2, 2, 4]
    _, s = _series(X, H, bits, policy, loop_group=4)
    for g in range(2):
        _, sg = _series(X[4 * g:4 * g + 4], H, bits[4 * g:4 * g + 4], policy)
        for r in range(4):
            _same(s, 4 * g + r, sg, r)
            anchor = 3 if policy == LAST else 0
            if r != anchor:
                assert np.array_equal(s.alpha[4 * g + r], sg.alpha[r])


def test_one_loop_groups_quantize_every_loop_directly():
    """loop_group = 1: every loop is its own anchor, i.e. plain group quantization."""
    X, H = _inputs(3)
    bits = [2, 4, 2]
    _, s = _series(X, H, bits, LAST, loop_group=1)
    for r in range(3):
        _, s1 = _series(X[r:r + 1], H, [bits[r]], LAST)
        _same(s, r, s1, 0)


def test_first_loop_mirrors_last_loop():
    """First-loop over loops 1..L = Last-loop over the loops in reverse order."""
    X, H = _inputs(4)
    bits = [4, 2, 2, 4]
    _, sf = _series(X, H, bits, FIRST)
    _, sl = _series(X[::-1].copy(), H, bits[::-1], LAST)
    for r in range(4):
        _same(sf, r, sl, 3 - r)
        if r != 0:
            assert np.array_equal(sf.alpha[r], sl.alpha[3 - r])


def test_first_loop_reconstruction_formula():
    """zhat_r = alpha_r A_1 + D(c_r) with A_1 the first loop's reconstruction (§3.2)."""
    X, H = _inputs(4)
    cfg, s = _series(X, H, [2, 2, 2, 4], FIRST)
    A = O.reconstruct(s, 0)
    for r in range(1, 4):
        zr = O.reconstruct(s, r)
        # the residual part alone: a loop-r series with alpha = 0 has the same D(c_r)
        al = O.f16_decode(s.alpha[r])
        res = zr - al[:, None] * A
        grp = res.reshape(T, -1, 32)
        meta = O.f16_decode(s.meta[r].reshape(-1)).reshape(T, -1, 2)
        codes = (grp - meta[:, :, :1]) / np.where(meta[:, :, 1:] > 0, meta[:, :, 1:], 1)
        assert np.allclose(codes, np.round(codes), atol=1e-9)      # integral codes: residual = o + s c


def test_grouped_chain_restarts_at_each_group():
    """Previous-loop within groups: the first loop of each group is an anchor (no alpha)."""
    X, H = _inputs(8)
    cfg, s = _series(X, H, [4, 2, 2, 2] * 2, PREV, loop_group=4)
    assert cfg.anchor(5) == 4 and cfg.anchor(3) == 0
    _, s4 = _series(X[4:5], H, [4], LAST)
    _same(s, 4, s4, 0)
