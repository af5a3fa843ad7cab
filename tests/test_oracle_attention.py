"""Pins for the attention oracles (paper §4.1, §4.2 Decode, App. G.2
'Reconstruction and attention', §5.3 BF16 baseline)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth


def _setup(bits, policy, T=53, D=64, head=1, identity=False):
    w = synth.WORKLOADS["tiny"]
    X = synth.kv(w, 0, 0, T + 1)                       # last token plays the current one
    Xk = synth.bits16(X[0, :, 0, head])
    Xv = synth.bits16(X[1, :, 0, head])
    if identity:
        HK = HV = np.eye(D, dtype=np.float32)
    else:
        HK = synth.rotation(w, 0, 0).numpy()[head]
        HV = synth.rotation(w, 0, 1).numpy()[head]
    cfg = O.Config(D=D, bits=list(bits), policy=policy)
    ks = O.quantize_series(cfg, Xk[:, :T], HK, diagnostics=False)
    vs = O.quantize_series(cfg, Xv[:, :T], HV, diagnostics=False)
    q = synth.bits16(synth.query(w, 0, 0, 0)[0, head])
    return cfg, Xk, Xv, HK, HV, ks, vs, q


def _textbook(qd, K, V, scale):
    s = scale * (K @ qd)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


@pytest.mark.parametrize("policy,bits", [(O.LAST_LOOP, (2, 2, 2, 4)), (O.LAST_LOOP, (2, 2, 4, 4)),
                                         (O.PREV_LOOP, (4, 4, 2, 2))])
def test_folded_attention_equals_bruteforce(policy, bits):
    """q' = HK q against rotated keys and one inverse V rotation equals attention
    on explicitly reconstructed Khat = HK^T zhat, Vhat = HV^T zhat."""
    cfg, Xk, Xv, HK, HV, ks, vs, q = _setup(bits, policy)
    T = ks.T
    for r in range(cfg.L):
        kc, vc = Xk[r, T], Xv[r, T]
        for Tp in (0, 1, 17, T):
            a = O.attend(ks, vs, r, Tp, HK, HV, q, kc, vc, 0.125)
            b = O.attend_bruteforce(ks, vs, r, Tp, HK, HV, q, kc, vc, 0.125)
            assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


def test_empty_cache_returns_current_value():
    cfg, Xk, Xv, HK, HV, ks, vs, q = _setup((2, 2, 2, 4), O.LAST_LOOP)
    out = O.attend(ks, vs, 1, 0, HK, HV, q, Xk[1, 5], Xv[1, 5], 0.125)
    assert np.array_equal(out, O.bf16_decode(Xv[1, 5]))


@pytest.mark.parametrize("identity", [True, False])
def test_16bit_attention_matches_textbook_on_inputs(identity):
    cfg, Xk, Xv, HK, HV, ks, vs, q = _setup((16, 16, 16, 16), O.LAST_LOOP, identity=identity)
    T = ks.T
    qd = O.bf16_decode(q)
    for r in range(cfg.L):
        K = O.bf16_decode(Xk[r, :T + 1])
        V = O.bf16_decode(Xv[r, :T + 1])
        ref = _textbook(qd, K, V, 0.125)
        got = O.attend(ks, vs, r, T, HK, HV, q, Xk[r, T], Xv[r, T], 0.125)
        assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_bf16_oracle_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    D, T = 96, 77
    K = synth.bits16(torch.randn(T + 1, D).to(torch.bfloat16))
    V = synth.bits16(torch.randn(T + 1, D).to(torch.bfloat16))
    q = synth.bits16(torch.randn(D).to(torch.bfloat16))
    scale = 1 / np.sqrt(D)
    got = O.attend_bf16(K[:T], V[:T], q, K[T], V[T], scale)
    t = lambda a: torch.from_numpy(O.bf16_decode(a))
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q)[None, None, None], t(K)[None, None], t(V)[None, None], scale=scale)[0, 0, 0].numpy()
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # large logits stay finite (max-subtracted softmax)
    big = O.attend_bf16(K[:T], V[:T], q, K[T], V[T], 300.0)
    assert np.all(np.isfinite(big))
