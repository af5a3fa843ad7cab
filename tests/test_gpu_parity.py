"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small and ragged shapes: whole caches and every output are compared. The
full-size workloads are covered in test_gpu_fullsize.py on sampled outputs.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_quantize_amd as rq
import oracle as O
import synth
from rq_parity import (TOL_ATTN, assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare,
                       inputs, log, max_rel_err, oracle_attention, oracle_layer, u16)

pytestmark = pytest.mark.gpu

LAST, PREV = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP


@pytest.mark.parametrize("policy,bits", [(LAST, (2, 2, 2, 4)), (LAST, (2, 2, 4, 4)), (PREV, (4, 4, 2, 2))])
def test_tiny_append_and_decode(policy, bits):
    w = synth.WORKLOADS["tiny"]
    T = w.T
    X, rk, rv = inputs(w, T + 1)
    label = f"tiny policy={policy} bits={bits}"
    log(f"{label}: append {T} tokens")
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, bits, policy, T)
    assert_cache_parity(compare_cache(cache, series, T), label)
    decode_and_compare(w, X, rk, rv, cache, series, [T], range(4), label)


def test_decode_mode_appends_match_bulk():
    """Token-by-token appends at increasing positions give the same cache as the oracle."""
    w = synth.WORKLOADS["tiny"].with_(batch=2)
    T = 70
    X, rk, rv = inputs(w, T + 1, batch=2)
    log("decode-mode appends")
    cache = build_gpu_layer(X, rk, rv, w.bits, LAST, T_max=T + 5, T=T, steps_of_one=9)
    series = oracle_layer(X, rk, rv, w.bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "decode-mode appends")


@pytest.mark.parametrize("wname,D,policy,chunk", [
    ("huginn_4k", 96, PREV, 3),     # eight loops: two per wave, a chain across waves and barriers
    ("tiny", 64, LAST, 8),          # the largest few-token append
    ("tiny", 64, LAST, 9),          # the smallest bulk append
    ("ouro_16k", 128, PREV, 2),
])
def test_few_token_appends(wname, D, policy, chunk):
    """Appends of a few tokens per call (the per-token store path) against the oracle."""
    w = synth.WORKLOADS[wname].with_(batch=3, heads=2, D=D)
    T = 41
    X, rk, rv = inputs(w, T, batch=3)
    bits = w.chained_bits if policy == PREV else w.bits
    label = f"{wname} D{D} policy={policy} chunks of {chunk}"
    log(label)
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 3, T=T, steps_of_one=T - 5, chunk=chunk)
    series = oracle_layer(X, rk, rv, bits, policy, T)
    assert_cache_parity(compare_cache(cache, series, T), label)


def test_ragged_lengths_and_edges():
    """Per-sequence lengths 0, 1, a tile boundary, a split boundary + 1 and a long
    ragged one; every loop; the current token always joins the softmax."""
    w = synth.WORKLOADS["tiny"].with_(batch=5, heads=3, D=128, nb=128, outliers=4)
    T = 700
    X, rk, rv = inputs(w, T + 1, batch=5)
    cache = build_gpu_layer(X, rk, rv, (2, 2, 4, 4), LAST, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, (2, 2, 4, 4), LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "ragged cache")
    d = cache.desc
    from_plan = rq.workspace_bytes(d)
    assert from_plan > 0
    lens = [0, 1, 32, 129, 699]
    decode_and_compare(w, X, rk, rv, cache, series, lens, range(4), "ragged")


def test_partial_and_combine():
    """The two halves of decode_attn reproduce it exactly, and the documented
    partial layout, merged in fp64 on the host with the oracle's current-token
    score, gives the oracle's output."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=3, D=128, nb=128)
    T = 900
    X, rk, rv = inputs(w, T + 1, batch=2)
    cache = build_gpu_layer(X, rk, rv, (2, 2, 4, 4), LAST, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, (2, 2, 4, 4), LAST, T)
    d = cache.desc
    B, H, D = 2, 3, 128
    lens = [T, 0]
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    unit, nsplit = rq.split_plan(d)
    scale = 1.0 / math.sqrt(D)
    for r in (0, 3):
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        ws1, ws2 = rq.alloc_workspace(d), rq.alloc_workspace(d)
        full = torch.empty(B, H, D, device="cuda")
        split = torch.empty(B, H, D, device="cuda")
        log(f"partial/combine loop {r}")
        rq.decode_attn(cache, r, q, kc, vc, past, scale, full, ws1)
        rq.decode_attn_partial(cache, r, q, past, scale, ws2)
        torch.cuda.synchronize()
        part = ws2[:B * H * nsplit * (D + 4) * 4].view(torch.float32).view(B, H, nsplit, D + 4).double().cpu()
        rq.decode_combine(d, cache.rot[1], q, kc, vc, past, scale, split, ws2)
        torch.cuda.synchronize()
        assert torch.equal(full, split)
        # host merge of the documented partials
        Hv = rv.double().numpy()
        qn, kn, vn = u16(q), u16(kc), u16(vc)
        units = [(b, h) for b in range(B) for h in range(H)]
        ref = oracle_attention(series, units, r, lens, rk, rv, q, kc, vc, scale)
        l2e = 1.0 / math.log(2.0)
        worst = 0.0
        for b, h in units:
            used = max(1, -(-lens[b] // rq.slot_len(lens[b], nsplit, unit)))
            P = part[b, h, :used].numpy()
            xq, xk, xv = O.bf16_decode(qn[b, h]), O.bf16_decode(kn[b, h]), O.bf16_decode(vn[b, h])
            xc = float(xq @ xk) * scale * l2e
            m = max([xc] + [float(v) for v in P[:, 0]])
            wts = np.where(P[:, 0] == -np.inf, 0.0, np.exp2(P[:, 0] - m))
            l = float(wts @ P[:, 1]) + 2.0 ** (xc - m)
            acc = Hv[h].T @ (wts @ P[:, 4:]) + 2.0 ** (xc - m) * xv
            o = acc / l
            worst = max(worst, np.abs(o - ref[(b, h)]).max() / np.abs(ref[(b, h)]).max())
        log(f"partial/combine loop {r}: host merge max rel err {worst:.3e}")
        assert worst <= TOL_ATTN


def test_huginn_shape_d96_eight_loops():
    w = synth.WORKLOADS["huginn_4k"].with_(batch=2, heads=3)
    T = 333
    X, rk, rv = inputs(w, T + 1, batch=2)
    cache = build_gpu_layer(X, rk, rv, w.bits, LAST, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, w.bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "d96 L8")
    decode_and_compare(w, X, rk, rv, cache, series, [T, 200], range(8), "d96 L8")


def test_uniform_int2_d128():
    w = synth.WORKLOADS["ouro_int2_4k"].with_(heads=4)
    T = 515
    X, rk, rv = inputs(w, T + 1)
    cache = build_gpu_layer(X, rk, rv, w.bits, LAST, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, w.bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "int2 d128")
    decode_and_compare(w, X, rk, rv, cache, series, [T], range(4), "int2 d128")


def test_bf16_decode_ragged():
    w = synth.WORKLOADS["tiny"].with_(batch=3, heads=2, D=128, nb=128)
    T = 600
    X, rk, rv = inputs(w, T + 1, batch=3)
    B, H, D = 3, 2, 128
    lens = [0, 77, 600]
    scale = 1.0 / math.sqrt(D)
    for r in range(4):
        d = rq.make_desc(B, H, D, (2, 2, 2, 4), T + 1)
        kcache = X[0, r].contiguous()
        vcache = X[1, r].contiguous()
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        out = torch.empty(B, H, D, device="cuda")
        ws = rq.alloc_workspace(d)
        past = torch.tensor(lens, dtype=torch.int32, device="cuda")
        log(f"bf16 loop {r}")
        rq.decode_attn_bf16(d, kcache, vcache, q, kc, vc, past, scale, out, ws)
        torch.cuda.synchronize()
        K, V = u16(kcache), u16(vcache)
        qn, kn, vn = u16(q), u16(kc), u16(vc)
        ref = {(b, h): O.attend_bf16(K[b, h, :lens[b]], V[b, h, :lens[b]], qn[b, h], kn[b, h], vn[b, h], scale)
               for b in range(B) for h in range(H)}
        err = max_rel_err(out, ref)
        log(f"bf16 loop {r} max rel err {err:.3e}")
        assert err <= TOL_ATTN


def test_device_error_flags():
    """Appends past capacity are dropped and flagged; lengths beyond capacity are clamped and flagged."""
    w = synth.WORKLOADS["tiny"]
    T_max = 40
    X, rk, rv = inputs(w, 64)
    d = rq.make_desc(1, 2, 64, w.bits, T_max)
    cache = rq.LayerCache.allocate(d, rk, rv)
    for kv in range(2):                       # never-written positions hold zeros, not garbage
        for r in range(d.loops):
            cache.codes[kv][r].zero_()
            cache.meta[kv][r].zero_()
            if cache.alpha[kv][r] is not None:
                cache.alpha[kv][r].zero_()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.tensor([30], dtype=torch.int32, device="cuda")
    log("device error flags: append past capacity")
    rq.quantize_append(cache, X[..., :20, :].contiguous(), pos, 20, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & rq.DEVERR_CAPACITY
    # the 10 tokens that fit were written: compare them with the oracle on tokens 30..39
    series = oracle_layer(X[..., :10, :], rk, rv, w.bits, LAST, 10)
    shifted = rq.LayerCache(d, [[c[:, :, 30:40].contiguous() for c in cs] for cs in cache.codes],
                            [[m[:, :, 30:40].contiguous() for m in ms] for ms in cache.meta],
                            [[None if a is None else a[:, :, 30:40].contiguous() for a in as_] for as_ in cache.alpha],
                            cache.rot)
    assert_cache_parity(compare_cache(shifted, series, 10), "capacity edge")
    # the few-token path: 5 tokens at position 37, 3 fit
    err.zero_()
    pos = torch.tensor([37], dtype=torch.int32, device="cuda")
    log("device error flags: few-token append past capacity")
    rq.quantize_append(cache, X[..., 20:25, :].contiguous(), pos, 5, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & rq.DEVERR_CAPACITY
    series = oracle_layer(X[..., 20:23, :], rk, rv, w.bits, LAST, 3)
    tail = rq.LayerCache(d, [[c[:, :, 37:40].contiguous() for c in cs] for cs in cache.codes],
                         [[m[:, :, 37:40].contiguous() for m in ms] for ms in cache.meta],
                         [[None if a is None else a[:, :, 37:40].contiguous() for a in as_] for as_ in cache.alpha],
                         cache.rot)
    assert_cache_parity(compare_cache(tail, series, 3), "few-token capacity edge")
    err.zero_()
    ws = rq.alloc_workspace(d)
    out = torch.empty(1, 2, 64, device="cuda")
    q = synth.query(w, 0, 0, 0, device="cuda")
    past = torch.tensor([T_max + 7], dtype=torch.int32, device="cuda")
    log("device error flags: length past capacity")
    rq.decode_attn(cache, 0, q, X[0, 0, :, :, 0].contiguous(), X[1, 0, :, :, 0].contiguous(), past,
                   0.125, out, ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & rq.DEVERR_LENGTH
    assert torch.isfinite(out).all()
