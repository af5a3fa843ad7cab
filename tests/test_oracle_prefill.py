"""Pins for the prefill attention oracle (paper §4.2 "Prefill": each loop
computes causal attention over its BF16 prompt K/V before the prompt is
quantized into the cache).

Checked against: torch's causal scaled_dot_product_attention in fp64 (a
library routine the oracle does not call), the decode oracle's textbook
attention row by row (the last query of a prefix is a decode step), the
single-token case and the causal independence of each row from later tokens.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth


def _inputs(T, D, seed):
    g = torch.Generator().manual_seed(seed)
    Q = synth.bits16(torch.randn(T, D, generator=g).to(torch.bfloat16))
    K = synth.bits16((1.5 * torch.randn(T, D, generator=g)).to(torch.bfloat16))
    V = synth.bits16(torch.randn(T, D, generator=g).to(torch.bfloat16))
    return Q, K, V


@pytest.mark.parametrize("T,D", [(1, 64), (37, 64), (130, 96), (200, 128)])
def test_matches_torch_causal_sdpa(T, D):
    Q, K, V = _inputs(T, D, T + D)
    scale = 1.0 / np.sqrt(D)
    got = O.prefill_attend(Q, K, V, scale)
    q, k, v = (torch.from_numpy(O.bf16_decode(x)) for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                                           scale=scale)[0].numpy()
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_each_row_is_a_decode_step():
    """Row i attends to keys 0..i: the decode oracle over the cache K[:i] with the
    current token (k_i, v_i) gives the same row."""
    T, D = 50, 64
    Q, K, V = _inputs(T, D, 3)
    got = O.prefill_attend(Q, K, V, 0.1)
    for i in (0, 1, 17, T - 1):
        row = O.attend_bf16(K[:i], V[:i], Q[i], K[i], V[i], 0.1)
        assert np.abs(got[i] - row).max() <= 1e-13 * np.abs(row).max()


def test_first_row_is_first_value():
    Q, K, V = _inputs(9, 64, 5)
    got = O.prefill_attend(Q, K, V, 0.125)
    assert np.array_equal(got[0], O.bf16_decode(V[0]))


def test_rows_ignore_later_tokens():
    T, D = 40, 64
    Q, K, V = _inputs(T, D, 8)
    a = O.prefill_attend(Q, K, V, 0.125)
    Q2, K2, V2 = (x.copy() for x in (Q, K, V))
    rng = np.random.default_rng(0)
    for x in (Q2, K2, V2):
        x[25:] = rng.integers(0x3C00, 0x4000, size=x[25:].shape).astype(np.uint16)   # other bf16 values
    b = O.prefill_attend(Q2, K2, V2, 0.125)
    assert np.array_equal(a[:25], b[:25])
    assert not np.array_equal(a[25:], b[25:])
