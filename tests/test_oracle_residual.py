"""Pins for residual quantization with LS scaling (paper §3.2, §3.3, §3.4,
App. D, App. G.1) in both reference policies."""
import numpy as np
import pytest

import oracle as O
import synth


def _bf16(x):
    import torch
    return synth.bits16(torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


def _decode_bf16(h):
    return O.bf16_decode(h)


def _tiny_series(bits=(2, 2, 2, 4), policy=O.LAST_LOOP, T=40, kv=0, seed_head=0, D=64, nb=64):
    w = synth.WORKLOADS["tiny"]
    X = synth.bits16(synth.kv(w, 0, 0, T)[kv, :, 0, seed_head])          # [L][T][D]
    H = synth.rotation(w, 0, kv).numpy()[seed_head]
    cfg = O.Config(D=w.D, bits=list(bits), policy=policy)
    return cfg, X, H, O.quantize_series(cfg, X, H)


def _rotated(X, H):
    """Z[r][t] = H x in fp64 (numpy matmul; independent of the oracle)."""
    x = _decode_bf16(X)
    return np.einsum("ij,rtj->rti", H.astype(np.float64), x)


def _meta_scales(s, r):
    m = s.meta[r].astype(np.uint16)                      # [T][G][2]
    return O.f16_decode(m[..., 0]), O.f16_decode(m[..., 1])


def test_alpha_is_least_squares_solution():
    cfg, X, H, s = _tiny_series()
    Z = _rotated(X, H)
    A = O.reconstruct(s, cfg.anchor())                   # anchor reconstruction
    for r in range(cfg.L - 1):
        for t in range(s.T):
            sol, *_ = np.linalg.lstsq(A[t][:, None], Z[r, t], rcond=None)
            assert abs(s.alpha_pre[r, t] - sol[0]) <= 1e-12 * max(1.0, abs(sol[0]))
            # stored alpha is the fp16 (nearest-even) rounding of the exact one
            assert s.alpha[r][t] == np.float16(s.alpha_pre[r, t]).view(np.uint16)


def test_residual_orthogonal_to_anchor():
    cfg, X, H, s = _tiny_series()
    Z = _rotated(X, H)
    A = O.reconstruct(s, cfg.anchor())
    for r in range(cfg.L - 1):
        for t in range(s.T):
            e = Z[r, t] - s.alpha_pre[r, t] * A[t]
            assert abs(e @ A[t]) <= 1e-5 * np.linalg.norm(Z[r, t]) * np.linalg.norm(A[t])


@pytest.mark.parametrize("policy,bits", [(O.LAST_LOOP, (2, 2, 2, 4)), (O.LAST_LOOP, (2, 2, 4, 4)),
                                         (O.PREV_LOOP, (4, 4, 2, 2)), (O.PREV_LOOP, (4, 2, 2, 2))])
def test_reconstruction_error_bound(policy, bits):
    """|zhat_r - Z_r| <= s_r/2 elementwise: each loop's error is its own residual's
    quantization error, whatever the reference (anchor or chain)."""
    cfg, X, H, s = _tiny_series(bits, policy)
    Z = _rotated(X, H)
    g = cfg.groups()[0]
    for r in range(cfg.L):
        zh = O.reconstruct(s, r)
        _, sc = _meta_scales(s, r)
        bound = np.repeat(sc, g, axis=1) / 2 * (1 + 2 ** -20) + 1e-12 * np.abs(Z[r]).max()
        assert np.all(np.abs(zh - Z[r]) <= bound)


def test_anchor_only_loop_reads_anchor():
    cfg, X, H, s = _tiny_series()
    a = cfg.anchor()
    A = O.reconstruct(s, a)
    o, sc = _meta_scales(s, a)
    codes = np.stack([np.concatenate([O.unpack_group(s.codes[a][t, j * 16:(j + 1) * 16], 32, 4)
                                      for j in range(2)]) for t in range(s.T)])
    ref = np.repeat(o, 32, axis=1) + np.repeat(sc, 32, axis=1) * codes
    assert np.array_equal(A, ref)


def test_last_loop_reconstruction_formula():
    cfg, X, H, s = _tiny_series()
    A = O.reconstruct(s, cfg.anchor())
    for r in range(cfg.L - 1):
        o, sc = _meta_scales(s, r)
        codes = np.stack([np.concatenate([O.unpack_group(s.codes[r][t, j * 8:(j + 1) * 8], 32, 2)
                                          for j in range(2)]) for t in range(s.T)])
        deq = np.repeat(o, 32, axis=1) + np.repeat(sc, 32, axis=1) * codes
        al = O.f16_decode(s.alpha[r])[:, None]
        assert np.array_equal(O.reconstruct(s, r), al * A + deq)


def test_near_lossless_at_16_bits():
    cfg, X, H, s = _tiny_series(bits=(16, 16, 16, 16))
    Z = _rotated(X, H)
    x = _decode_bf16(X)
    for r in range(cfg.L):
        zh = O.reconstruct(s, r)
        xh = zh @ H.astype(np.float64)                  # Xhat = H^T zhat, row form
        nmse = np.sum((xh - x[r]) ** 2) / max(np.sum(x[r] ** 2), 1e-30)   # Table 1 NMSE definition
        assert nmse < 1e-9
        assert np.all(np.abs(zh - Z[r]) <= np.abs(Z[r]).max() * 2.0 ** -15)


def test_single_loop_is_plain_group_quantization():
    cfg, X, H, s = _tiny_series()
    cfg1 = O.Config(D=64, bits=[4], policy=O.LAST_LOOP)
    s1 = O.quantize_series(cfg1, X[3:4], H)
    Z = _rotated(X[3:4], H)
    for t in range(s1.T):
        for j in range(2):
            o16, s16, codes, *_ = O.group_quant(Z[0, t, 32 * j:32 * (j + 1)], 4)
            assert s1.meta[0][t, j].tolist() == [o16, s16]
            assert np.array_equal(s1.codes[0][t, 16 * j:16 * (j + 1)], O.pack_group(codes, 4))


def test_identity_rotation_quantizes_original_values():
    cfg, X, H, s = _tiny_series()
    I = np.eye(64, dtype=np.float32)
    sI = O.quantize_series(O.Config(D=64, bits=[4], policy=O.LAST_LOOP), X[3:4], I)
    x = _decode_bf16(X[3])
    for t in range(sI.T):
        o16, s16, codes, *_ = O.group_quant(x[t, :32], 4)
        assert sI.meta[0][t, 0].tolist() == [o16, s16]


def test_scaled_copy_and_zero_loops():
    """X_1 = k X_L gives alpha_1 = k * <Z_L, A>/|A|^2; X_2 = 0 gives alpha = 0 and an
    all-zero residual (s = 0, codes 0)."""
    rng = np.random.default_rng(0)
    T, D = 12, 64
    xl = rng.normal(size=(T, D)).astype(np.float32)
    xl_b = _bf16(xl)
    xl_d = _decode_bf16(xl_b)
    X = np.stack([_bf16(0.5 * xl_d), np.zeros((T, D), np.uint16), _bf16(2.0 * xl_d), xl_b])
    H = O.rotation(D, D, rng.choice([-1, 1], D).astype(np.int8)).astype(np.float32)
    for bits in [(2, 2, 2, 4), (16, 16, 16, 16)]:
        cfg = O.Config(D=D, bits=list(bits))
        s = O.quantize_series(cfg, X, H)
        A = O.reconstruct(s, 3)
        Zl = _rotated(X[3:4], H)[0]
        self_alpha = np.einsum("ti,ti->t", Zl, A) / np.einsum("ti,ti->t", A, A)
        assert np.allclose(s.alpha_pre[0], 0.5 * self_alpha, rtol=1e-12, atol=0)
        assert np.allclose(s.alpha_pre[2], 2.0 * self_alpha, rtol=1e-12, atol=0)
        if bits[3] == 16:
            assert np.all(np.abs(s.alpha_pre[0] - 0.5) < 1e-4)
        assert np.all(s.alpha_pre[1] == 0.0) and np.all(s.alpha[1] == 0)
        assert np.all(s.meta[1] == 0) and np.all(s.codes[1] == 0)


@pytest.mark.parametrize("b1,b2", [(4, 2), (2, 4), (4, 4)])
def test_two_loop_chain_mirrors_last_loop(b1, b2):
    """With two loops, Previous-loop on (X1, X2) is Last-loop on (X2, X1): same bytes."""
    cfg, X, H, _ = _tiny_series()
    Xp = X[[1, 3]]
    sp = O.quantize_series(O.Config(D=64, bits=[b1, b2], policy=O.PREV_LOOP), Xp, H)
    sl = O.quantize_series(O.Config(D=64, bits=[b2, b1], policy=O.LAST_LOOP), Xp[::-1].copy(), H)
    assert np.array_equal(sp.codes[0], sl.codes[1]) and np.array_equal(sp.codes[1], sl.codes[0])
    assert np.array_equal(sp.meta[0], sl.meta[1]) and np.array_equal(sp.meta[1], sl.meta[0])
    assert np.array_equal(sp.alpha[1], sl.alpha[0])


def test_chained_reconstruction_recurrence():
    cfg, X, H, s = _tiny_series((4, 4, 2, 2), O.PREV_LOOP)
    prev = O.reconstruct(s, 0)
    g = 32
    for r in range(1, cfg.L):
        b = cfg.bits[r]
        o, sc = _meta_scales(s, r)
        nb = g * b // 8
        codes = np.stack([np.concatenate([O.unpack_group(s.codes[r][t, j * nb:(j + 1) * nb], g, b)
                                          for j in range(2)]) for t in range(s.T)])
        deq = np.repeat(o, g, axis=1) + np.repeat(sc, g, axis=1) * codes
        cur = O.reconstruct(s, r)
        assert np.array_equal(cur, O.f16_decode(s.alpha[r])[:, None] * prev + deq)
        prev = cur


def test_alpha_tracks_generator_similarity():
    """Statistical sanity on the synthetic law (not a parity pin): with noise drawn
    independently of the anchor, the mean LS alpha of loop r is near s_r."""
    w = synth.WORKLOADS["tiny"]
    T = 256
    for kv in (0, 1):
        X = synth.bits16(synth.kv(w, 0, 0, T)[kv, :, 0, 0])
        H = synth.rotation(w, 0, kv).numpy()[0]
        s = O.quantize_series(O.Config(D=64, bits=[2, 2, 2, 4]), X, H)
        for r in range(3):
            assert abs(s.alpha_pre[r].mean() / w.sim(r + 1) - 1) < 0.03


def test_alpha_beyond_fp16_range_saturates():
    """A loop about 1e6 times its (small) anchor along the same direction: the exact LS
    coefficient overflows fp16, the stored one is 65504 and the residual is taken with it."""
    rng = np.random.default_rng(3)
    T, D = 6, 64
    base = rng.normal(size=(T, D)).astype(np.float32)
    anchor = _bf16(1e-4 * base)
    loop = _bf16(1e2 * O.bf16_decode(anchor).astype(np.float32) * 1e4)   # ~1e6 x the anchor
    X = np.stack([loop, anchor])
    H = np.eye(D, dtype=np.float32)
    s = O.quantize_series(O.Config(D=D, bits=[4, 4]), X, H)
    A = O.reconstruct(s, 1)
    Z = O.bf16_decode(loop)
    exact = np.einsum("td,td->t", Z, A) / np.einsum("td,td->t", A, A)      # numpy LS, no fp16
    assert np.all(np.abs(exact) > 65520.0)                                # fp16 would round to inf
    assert np.all(s.alpha[0] == np.float16(65504.0).view(np.uint16))
    assert np.allclose(s.alpha_pre[0], exact, rtol=1e-12)
    # the residual is quantized against alpha = 65504: reconstruction = 65504 A + D(c)
    o, sc = _meta_scales(s, 0)
    codes = np.stack([np.concatenate([O.unpack_group(s.codes[0][t, j * 16:(j + 1) * 16], 32, 4)
                                      for j in range(2)]) for t in range(T)])
    deq = np.repeat(o, 32, axis=1) + np.repeat(sc, 32, axis=1) * codes
    assert np.array_equal(O.reconstruct(s, 0), 65504.0 * A + deq)
    E = Z - 65504.0 * A
    assert np.all(np.abs(O.reconstruct(s, 0) - Z) <= np.repeat(sc, 32, axis=1) / 2 * (1 + 2 ** -20)
                  + 1e-9 * np.abs(E).max())
