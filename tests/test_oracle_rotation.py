"""Pins for the oracle's randomized Hadamard rotation (paper §2.2, App. G.2)."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O
import synth


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_matches_scipy(n):
    assert np.array_equal(O.sylvester(n), scipy.linalg.hadamard(n).astype(np.float64))


@pytest.mark.parametrize("D,nb", [(64, 64), (128, 128), (96, 32)])
def test_rotation_orthogonal(D, nb):
    rng = np.random.default_rng(D)
    sign = rng.choice([-1, 1], D).astype(np.int8)
    H = O.rotation(D, nb, sign)
    assert np.abs(H.T @ H - np.eye(D)).max() < 1e-14
    assert np.abs(H @ H.T - np.eye(D)).max() < 1e-14
    H32 = H.astype(np.float32).astype(np.float64)
    assert np.abs(H32.T @ H32 - np.eye(D)).max() < 1e-6          # fp32 storage keeps H^T H = I to 1e-6
    # block-diagonal structure and magnitudes 1/sqrt(nb)
    for i in range(D):
        for j in range(D):
            same = i // nb == j // nb
            assert (abs(abs(H[i, j]) - 1 / np.sqrt(nb)) < 1e-15) if same else H[i, j] == 0.0


def test_rotation_sign_is_column_scaling():
    D = 64
    sign = np.ones(D, np.int8)
    sign[5] = -1
    H = O.rotation(D, D, sign)
    W = scipy.linalg.hadamard(D) / 8.0
    W[:, 5] *= -1
    assert np.array_equal(H, W)


@pytest.mark.parametrize("name", ["tiny", "huginn_4k"])
def test_generator_rotation_matches_oracle_construction(name):
    w = synth.WORKLOADS[name]
    H = synth.rotation(w, 0, 1).numpy()
    sign = synth.rotation_signs(w, 0, 1).numpy()
    for h in range(w.heads):
        ref = O.rotation(w.D, w.block, sign[h]).astype(np.float32)
        assert np.array_equal(H[h], ref)
