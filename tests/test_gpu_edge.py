"""GPU parity (through the C ABI) against the CPU oracle on the method's edge cases.

Paper "KV Cache Quantization for Looped Transformers with 2-Bit Residuals":
§2.1 affine group quantization (constant groups give a zero scale), §3.2
"Scaling coefficient" (scaled copies give alpha = k; a zero loop or a zero
anchor give alpha = 0), §3.3 shared rotation (any orthogonal matrix, such as a
learned one, takes the Hadamard's place), §4.1 FP32 softmax and App. G.2
(reconstruction inside attention; sharp softmax distributions).

Inputs are built here from their own recipe (no generator of the method's
arithmetic); the oracle quantizes the very bf16 bytes the GPU consumed. Caches
are compared element by element (bit-exact fp16 metadata and alpha, codes
exact up to documented ties) and every decoded loop's output against the
oracle's attention over its own quantization.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import decode_attention_quantize_amd as rq
import oracle as O
import synth
from rq_parity import (TOL_ATTN, assert_cache_parity, build_gpu_layer, compare_cache, log, max_rel_err,
                       oracle_attention, oracle_layer, u16)

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP


def _bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, np.float64), dtype=torch.float64).to(torch.bfloat16)


def _grid_row(rng, D, g, bits):
    """A row whose groups of g lie exactly on a 2^bits-level grid o + s c (o, s multiples
    of 1/8, both ends used): the group quantizer reproduces it without error, and every
    value is exact in bf16 and fp16."""
    qmax = 2 ** bits - 1
    out = np.empty(D)
    for j in range(D // g):
        o = rng.integers(-16, 1) / 8.0
        s = rng.integers(1, 5) / 8.0
        c = rng.integers(0, qmax + 1, g)
        c[0], c[1] = 0, qmax
        rng.shuffle(c)
        out[j * g:(j + 1) * g] = o + s * c
    return out


KINDS = ("scaled_copies", "const_residual", "zero_anchor", "zero_loops", "all_zero", "const_anchor",
         "near_copies", "generic")


def degenerate_inputs(B, H, D, L, T, anchor, anchor_bits, seed):
    """bf16 [2][L][B][H][T][D]: token t of every series is of kind KINDS[t % len(KINDS)]
    (the anchor loop holds the reference, the other loops are built from it)."""
    rng = np.random.default_rng(seed)
    X = np.zeros((2, L, B, H, T, D))
    ks = [0.5, -1.0, 2.0, 0.75, -0.25, 1.0, 0.5, -2.0]
    for kv in range(2):
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    kind = KINDS[t % len(KINDS)]
                    A = np.zeros(D)
                    loops = np.zeros((L, D))
                    if kind == "scaled_copies":
                        A = _grid_row(rng, D, 32, anchor_bits)
                        for r in range(L):
                            loops[r] = ks[(r + t) % len(ks)] * A
                    elif kind == "const_residual":
                        A = _grid_row(rng, D, 32, anchor_bits)
                        A[32:64] = 0.0                     # a zero group of the anchor
                        for r in range(L):
                            loops[r] = A.copy()
                            # constant, not exact in fp16 (subnormal range, below its spacing)
                            loops[r][32:64] = float(_bf16([1.1e-6 * (r + 1)])[0])
                    elif kind == "zero_anchor":
                        loops = rng.normal(size=(L, D))
                    elif kind == "zero_loops":
                        A = rng.normal(size=D)
                    elif kind == "all_zero":
                        pass
                    elif kind == "const_anchor":
                        A = np.repeat(rng.integers(-24, 25, D // 32) / 4.0, 32)   # fp16-exact constants
                        loops = rng.normal(size=(L, D))
                    elif kind == "near_copies":
                        A = rng.normal(size=D)
                        loops = A[None, :] + 1e-3 * rng.normal(size=(L, D))
                    else:
                        A = rng.normal(size=D) * np.exp(0.5 * rng.normal(size=D))
                        loops = 0.85 * A[None, :] + 0.3 * rng.normal(size=(L, D))
                    X[kv, :, b, h, t] = loops
                    X[kv, anchor, b, h, t] = A
    return _bf16(X)


def rotation(kind, H, D, seed):
    """fp32 [H][D][D] orthogonal matrices: identity, signed permutation, random-sign
    Hadamard (block 32 for D = 96), or Q of a Gaussian matrix's QR factorization."""
    rng = np.random.default_rng(seed)
    out = np.zeros((H, D, D))
    for h in range(H):
        if kind == "identity":
            M = np.eye(D)
        elif kind == "perm":
            M = np.eye(D)[rng.permutation(D)] * rng.choice([-1.0, 1.0], D)[:, None]
        elif kind == "hadamard":
            nb = 32 if D == 96 else D
            W = scipy.linalg.hadamard(nb) / math.sqrt(nb)
            M = scipy.linalg.block_diag(*([W] * (D // nb))) * rng.choice([-1.0, 1.0], D)[None, :]
        else:
            M, _ = np.linalg.qr(rng.normal(size=(D, D)))
        out[h] = M
    return torch.from_numpy(out.astype(np.float32))


def _decode_all(cache, X, rk, rv, series, lens, label, q_scale=1.0, cur_scale=1.0, flags=None, seed=0):
    """Decode every loop with a random query (times q_scale) and a random current token
    (times cur_scale); return the worst relative error against the oracle."""
    d = cache.desc
    B, H, D, L = d.batch, d.heads, d.head_dim, d.loops
    g = torch.Generator().manual_seed(seed)
    ws = rq.alloc_workspace(d)
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    worst = 0.0
    for r in range(L):
        q = (torch.randn(B, H, D, generator=g, dtype=torch.float64) * q_scale).to(torch.bfloat16).cuda()
        kc = (torch.randn(B, H, D, generator=g, dtype=torch.float64) * cur_scale).to(torch.bfloat16).cuda()
        vc = (torch.randn(B, H, D, generator=g, dtype=torch.float64) * cur_scale).to(torch.bfloat16).cuda()
        out = torch.empty(B, H, D, device="cuda")
        rq.decode_attn(cache, r, q, kc, vc, past, scale, out, ws, flags=flags)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), (label, r)
        units = [(b, h) for b in range(B) for h in range(H)]
        ref = oracle_attention(series, units, r, lens, rk, rv, q, kc, vc, scale)
        err = max_rel_err(out, ref)
        worst = max(worst, err)
        log(f"{label}: loop {r} max rel err {err:.3e}")
        assert err <= TOL_ATTN, (label, r, err)
    return worst


CASES = [
    # D, policy, bits, groups, rotation
    (64, LAST, (2, 2, 2, 4), 32, "identity"),
    (64, PREV, (4, 4, 2, 2), 32, "perm"),
    (64, FIRST, (4, 2, 2, 2), 32, "hadamard"),
    (96, LAST, (2, 2, 4, 4), 32, "identity"),
    (96, PREV, (4, 2, 2, 2), 32, "hadamard"),
    (96, FIRST, (4, 2, 4, 2), 32, "perm"),
    (128, LAST, (2, 2, 4, 4), 32, "identity"),
    (128, LAST, (2, 2, 2, 2), 32, "hadamard"),
    (128, LAST, (2, 2, 4, 4), (16, 16, 32, 32), "identity"),
    (128, PREV, (4, 4, 2, 2), 32, "identity"),
    (128, FIRST, (4, 2, 2, 4), (32, 16, 16, 32), "perm"),
]


@pytest.mark.parametrize("D,policy,bits,groups,rot", CASES,
                         ids=[f"D{c[0]}-p{c[1]}-{''.join(map(str, c[2]))}-g{c[3] if c[3] == 32 else 'mix'}-{c[4]}"
                              for c in CASES])
def test_degenerate_groups_and_loops(D, policy, bits, groups, rot):
    """Constant groups (fp16-exact: s = 0; inexact: a subnormal scale), scaled copies
    (alpha = k and a zero residual), an all-zero loop (alpha = 0), an all-zero anchor
    (|A| = 0, so alpha = 0 and the residual is the loop itself), near-copies and generic
    tokens, interleaved in one cache; the bulk store, then few-token stores; every loop
    decoded at two lengths."""
    B, H, L, T = 2, 2, 4, 2 * 8 * 16 + 5
    G = L
    anchor = G - 1 if policy == LAST else 0
    X = degenerate_inputs(B, H, D, L, T + 1, anchor, bits[anchor], seed=D + 7 * policy).cuda()
    rk, rv = rotation(rot, H, D, seed=1), rotation(rot, H, D, seed=2)
    label = f"edge D{D} policy={policy} bits={bits} groups={groups} rot={rot}"
    log(label)
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T, steps_of_one=7, chunk=3, groups=groups)
    series = oracle_layer(X, rk, rv, bits, policy, T, groups=groups)
    stats = compare_cache(cache, series, T)
    assert_cache_parity(stats, label)
    if rot == "identity" and policy == LAST:
        # the structure really reached the quantizer: exact copies give exact alphas
        s = series[(0, 0, 0)]
        t0 = KINDS.index("scaled_copies")
        assert s.alpha_pre[0, t0] in (0.5, -1.0, 2.0, 0.75, -0.25, 1.0, -2.0)
        assert np.all(s.meta[0][KINDS.index("all_zero")] == 0)
    _decode_all(cache, X, rk, rv, series, [T, T - 37], label, seed=D)


def test_fp16_range_extremes():
    """Groups near the top of the fp16 range (values to about 6e4) and in its subnormal
    range (about 1e-6): offsets and scales at the fp16 extremes, exact or subnormal, with
    no saturation; queries scaled so that the logits stay moderate."""
    B, H, D, L, T = 1, 2, 128, 4, 160
    rng = np.random.default_rng(11)
    rk, rv = rotation("identity", H, D, 0), rotation("identity", H, D, 0)
    for name, mag in (("large", 5000.0), ("tiny", 1.0 / 1048576.0)):
        # grid rows shifted into [-11.5, 0] (offsets toward -6e4 at the large magnitude)
        base = np.stack([_grid_row(rng, D, 32, 4) - 9.5 for _ in range(2 * B * H * (T + 1))])
        base = base.reshape(2, 1, B, H, T + 1, D)
        noise = rng.normal(size=(2, L, B, H, T + 1, D)) * 0.25
        X = _bf16(mag * (base * np.array([0.6, 0.7, 0.8, 1.0])[None, :, None, None, None, None] + noise)).cuda()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        bits = (2, 2, 4, 4)
        d = rq.make_desc(B, H, D, bits, T + 1)
        cache = rq.LayerCache.allocate(d, rk, rv)
        rq.quantize_append(cache, X[..., :T, :].contiguous(), torch.zeros(B, dtype=torch.int32, device="cuda"), T,
                           dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, name
        series = oracle_layer(X, rk, rv, bits, LAST, T)
        m = np.concatenate([O.f16_decode(s.meta[r]).ravel() for s in series.values() for r in range(L)])
        if name == "large":
            assert np.abs(m).max() > 3e4
        else:
            assert np.any((m != 0) & (np.abs(m) < 2.0 ** -14))       # subnormal offsets or scales
        assert_cache_parity(compare_cache(cache, series, T), f"fp16 extremes {name}")
        _decode_all(cache, X, rk, rv, series, [T], f"fp16 extremes {name}", q_scale=1.0 / mag, cur_scale=mag,
                    seed=3)


def test_saturation_flag_and_parity():
    """Inputs beyond the fp16 range: offsets, scales and an LS coefficient that would round
    to infinity are stored as +-65504, the cache stays finite and equal to the oracle's
    (the same saturating rule), RQ_DEVERR_RANGE is raised, and decode stays finite."""
    B, H, D, L, T = 1, 1, 64, 2, 40
    rng = np.random.default_rng(5)
    X = np.zeros((2, L, B, H, T, D))
    for t in range(T):
        if t % 2 == 0:                 # a group below -65504 and a group range past 15 * 65504
            X[:, 1, 0, 0, t] = rng.normal(size=D) * 10.0
            X[:, 1, 0, 0, t, :32] = np.linspace(-90000.0, 30000.0, 32)
            X[:, 1, 0, 0, t, 32:] = np.linspace(-10.0, 1.2e6, 32)
            X[:, 0, 0, 0, t] = 0.5 * X[:, 1, 0, 0, t] + rng.normal(size=D)
        else:                          # a tiny anchor and a loop 1e6 times larger: alpha overflows
            a = rng.normal(size=D) * 1e-4
            X[:, 1, 0, 0, t] = a
            X[:, 0, 0, 0, t] = float(1e6) * a
    Xb = _bf16(X).cuda()
    rk, rv = rotation("identity", H, D, 0), rotation("identity", H, D, 0)
    bits = (4, 4)
    d = rq.make_desc(B, H, D, bits, T)
    cache = rq.LayerCache.allocate(d, rk, rv)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rq.quantize_append(cache, Xb[..., :T - 4, :].contiguous(), torch.zeros(B, dtype=torch.int32, device="cuda"),
                       T - 4, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & rq.DEVERR_RANGE
    err.zero_()
    rq.quantize_append(cache, Xb[..., T - 4:, :].contiguous(), torch.full((B,), T - 4, dtype=torch.int32,
                                                                          device="cuda"), 4, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & rq.DEVERR_RANGE                     # the few-token path flags too
    series = oracle_layer(Xb, rk, rv, bits, LAST, T)
    s = series[(0, 0, 0)]
    assert np.any(s.meta[1] == np.float16(-65504.0).view(np.uint16))
    assert np.any(s.alpha[0] == np.float16(65504.0).view(np.uint16))
    for kv in range(2):
        for r in range(L):
            assert torch.isfinite(cache.meta[kv][r].view(torch.float16).float()).all()
    assert_cache_parity(compare_cache(cache, series, T), "saturation")
    _decode_all(cache, Xb, rk, rv, series, [T - 1], "saturation", q_scale=2e-6, seed=4)


@pytest.mark.parametrize("D,policy", [(64, LAST), (96, PREV), (128, LAST), (128, FIRST)])
def test_qr_rotation_append_and_decode(D, policy):
    """A dense orthogonal rotation (Q of a Gaussian QR factorization, rounded to fp32), as
    a learned rotation would be, in place of the randomized Hadamard: the whole cache and
    every loop's output against the oracle, which applies the same fp32 matrix."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=3, D=D, nb=32 if D == 96 else D, outliers=3)
    T = 300
    X = synth.kv(w, 0, 0, T + 1, device="cuda", batch=2)
    rk, rv = rotation("qr", 3, D, seed=D), rotation("qr", 3, D, seed=D + 1)
    bits = (2, 2, 4, 4) if policy == LAST else (4, 4, 2, 2)
    label = f"qr rotation D{D} policy={policy}"
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T, steps_of_one=5)
    series = oracle_layer(X, rk, rv, bits, policy, T)
    assert_cache_parity(compare_cache(cache, series, T), label)
    _decode_all(cache, X, rk, rv, series, [T, 77], label, seed=D)


def test_sharp_logits_query_precision():
    """Softmax sharpness against the fixed-point query: at 16k cached tokens (the
    benchmark's plan and inputs, two series), queries scaled x1 .. x16 sharpen the
    logits; the 21-bit query (RQ_FLAG_PRECISE_QUERY) stays within the bar at every scale,
    and the default 14-bit query within it at the unscaled logits. Errors are logged per
    scale for both."""
    w = synth.WORKLOADS["ouro_16k"].with_(batch=1, heads=2)
    T = w.T
    X = synth.kv(w, 0, 0, T + 1, device="cuda", batch=1)
    rk, rv = synth.rotation(w, 0, 0), synth.rotation(w, 0, 1)
    d = rq.make_desc(1, 2, 128, list(w.bits), T + 64)
    cache = rq.LayerCache.allocate(d, rk, rv)
    rq.quantize_append(cache, X[..., :T, :].contiguous(), torch.zeros(1, dtype=torch.int32, device="cuda"), T)
    torch.cuda.synchronize()
    series = oracle_layer(X, rk, rv, w.bits, LAST, T)
    ws = rq.alloc_workspace(d)
    past = torch.tensor([T], dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(128)
    units = [(0, 0), (0, 1)]
    table = []
    for r in (0, 2):
        q0 = synth.query(w, 0, r, 0, device="cpu", batch=1).double()
        kc = X[0, r, :, :, T].contiguous()
        vc = X[1, r, :, :, T].contiguous()
        for mult in (1, 2, 4, 8, 16):
            q = (q0 * mult).to(torch.bfloat16).cuda()
            ref = oracle_attention(series, units, r, [T], rk, rv, q, kc, vc, scale)
            errs = {}
            for name, flags in (("14-bit", 0), ("21-bit", rq.FLAG_PRECISE_QUERY)):
                out = torch.empty(1, 2, 128, device="cuda")
                rq.decode_attn(cache, r, q, kc, vc, past, scale, out, ws, flags=flags)
                torch.cuda.synchronize()
                errs[name] = max_rel_err(out, ref)
            log(f"sharp logits loop {r} q x{mult}: 14-bit {errs['14-bit']:.3e} 21-bit {errs['21-bit']:.3e}")
            table.append((r, mult, errs["14-bit"], errs["21-bit"]))
            assert errs["21-bit"] <= TOL_ATTN, (r, mult, errs)
            if mult == 1:
                assert errs["14-bit"] <= TOL_ATTN, (r, mult, errs)
    # the 21-bit query is at least 16 times closer wherever the 14-bit error is visible
    for r, mult, e14, e21 in table:
        if e14 > 1e-4:
            assert e21 <= e14 / 16, (r, mult, e14, e21)
