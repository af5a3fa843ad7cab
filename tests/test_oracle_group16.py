"""Oracle pins for INT2 groups of 16 channels (paper §5 "Quantization setup":
g = 16 for uniform INT2 and as the second INT2 group size of Table 2; App. A.3
effective bit widths), alone and mixed with INT4 groups of 32 in one plan.

Each pin checks the oracle against something it does not compute the same way:
the plain group quantizer applied to explicit 16-channel slices of H x (numpy
rotation), the per-element error bound of each group's own scale, the
reconstruction formula written out with the layout rule, and brute-force
attention on explicitly reconstructed keys and values.
"""
import numpy as np
import pytest

import oracle as O
import synth


def _series(bits, groups, policy=O.LAST_LOOP, T=37, kv=0, head=1):
    w = synth.WORKLOADS["tiny"]
    X = synth.bits16(synth.kv(w, 0, 0, T + 1)[kv, :, 0, head])          # [L][T+1][D]
    H = synth.rotation(w, 0, kv).numpy()[head]
    L = len(bits)
    cfg = O.Config(D=w.D, bits=list(bits), group=list(groups), policy=policy)
    return cfg, X[:L], H, O.quantize_series(cfg, X[:L, :T], H)


def _rotated(X, H):
    return np.einsum("ij,rtj->rti", H.astype(np.float64), O.bf16_decode(X))


def _unpack_row(row, D, bits, g):
    n = g * bits // 8
    return np.concatenate([O.unpack_group(row[j * n:(j + 1) * n], g, bits) for j in range(D // g)])


def test_single_loop_is_plain_group16_quantization():
    """One INT2 loop at g = 16: each 16-channel slice of H x is the plain group quantizer's."""
    cfg, X, H, s = _series((2,), (16,))
    Z = _rotated(X, H)
    assert s.meta[0].shape[1:] == (4, 2)                  # D/16 groups of (offset, scale)
    for t in range(s.T):
        for j in range(4):
            o16, s16, codes, *_ = O.group_quant(Z[0, t, 16 * j:16 * (j + 1)], 2)
            assert s.meta[0][t, j].tolist() == [o16, s16]
            assert np.array_equal(s.codes[0][t, 4 * j:4 * (j + 1)], O.pack_group(codes, 2))


@pytest.mark.parametrize("policy,bits,groups", [
    (O.LAST_LOOP, (2, 2, 2, 4), (16, 16, 16, 32)),
    (O.LAST_LOOP, (2, 2, 2, 2), (16, 16, 16, 16)),
    (O.PREV_LOOP, (4, 2, 2, 2), (32, 16, 16, 16)),
    (O.FIRST_LOOP, (4, 2, 2, 2), (32, 16, 16, 16)),
])
def test_error_within_half_a_step_of_each_group(policy, bits, groups):
    """|zhat_r - Z_r| <= s_{r,group}/2 for every element, with the group of that loop's size."""
    cfg, X, H, s = _series(bits, groups, policy)
    Z = _rotated(X[:, :s.T], H)
    for r in range(cfg.L):
        zh = O.reconstruct(s, r)
        sc = O.f16_decode(s.meta[r][..., 1].astype(np.uint16))
        assert sc.shape[1] == cfg.D // groups[r]
        bound = np.repeat(sc, groups[r], axis=1) / 2 * (1 + 2 ** -20) + 1e-12 * np.abs(Z[r]).max()
        assert np.all(np.abs(zh - Z[r]) <= bound)


def test_last_loop_reconstruction_with_two_group_sizes():
    """zhat_r = alpha_r A + o + s c with A the INT4 g32 anchor and the INT2 g16 residual
    written out from the layout rule."""
    cfg, X, H, s = _series((2, 2, 2, 4), (16, 16, 16, 32))
    A = O.reconstruct(s, 3)
    for r in range(3):
        o = O.f16_decode(s.meta[r][..., 0].astype(np.uint16))
        sc = O.f16_decode(s.meta[r][..., 1].astype(np.uint16))
        codes = np.stack([_unpack_row(s.codes[r][t], cfg.D, 2, 16) for t in range(s.T)])
        deq = np.repeat(o, 16, axis=1) + np.repeat(sc, 16, axis=1) * codes
        al = O.f16_decode(s.alpha[r])[:, None]
        assert np.array_equal(O.reconstruct(s, r), al * A + deq)


def test_group16_residual_codes_use_all_levels():
    """Each 16-channel residual group maps its min and max to levels 0 and 3 (up to the
    fp16 rounding of offset and scale): the extremes of the group, not of its 32-block."""
    cfg, X, H, s = _series((2, 2, 2, 4), (16, 16, 16, 32), T=60)
    lo = hi = n = 0
    for r in range(3):
        for t in range(s.T):
            c = _unpack_row(s.codes[r][t], cfg.D, 2, 16).reshape(-1, 16)
            lo += int(np.sum(c.min(axis=1) == 0))
            hi += int(np.sum(c.max(axis=1) == 3))
            n += c.shape[0]
    assert lo == n and hi >= 0.97 * n


@pytest.mark.parametrize("policy,bits,groups", [
    (O.LAST_LOOP, (2, 2, 2, 4), (16, 16, 16, 32)),
    (O.PREV_LOOP, (2, 2, 2, 2), (16, 16, 16, 16)),
])
def test_folded_attention_equals_bruteforce_group16(policy, bits, groups):
    cfg, X, H, s = _series(bits, groups, policy, kv=0)
    w = synth.WORKLOADS["tiny"]
    Xv = synth.bits16(synth.kv(w, 0, 0, s.T + 1)[1, :, 0, 1])
    HV = synth.rotation(w, 0, 1).numpy()[1]
    vs = O.quantize_series(cfg, Xv[:, :s.T], HV)
    q = synth.bits16(synth.query(w, 0, 0, 0)[0, 1])
    for r in range(cfg.L):
        for Tp in (1, 16, s.T):
            a = O.attend(s, vs, r, Tp, H, HV, q, X[r, s.T], Xv[r, s.T], 0.125)
            b = O.attend_bruteforce(s, vs, r, Tp, H, HV, q, X[r, s.T], Xv[r, s.T], 0.125)
            assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()
