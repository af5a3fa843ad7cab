"""GPU parity at the benchmark's full sizes and launch configuration.

The 16k workload (B8, H16, D128, 4 loops, 16384 cached tokens, 64 decode
steps, plan [2,2,4,4]; chained comparator [4,4,2,2]) is built exactly as the
benchmark builds it: the same cache descriptor (token capacity 16384 + 64, so
the same split plan and grid), a bulk store of the prompt tokens and one
single-token store per decode step. Decode runs at steps 0 and 63 with the
benchmark's queries and current tokens.

Layer 0 is checked for every (batch, head): the whole cache (codes, fp16
metadata and LS coefficients of every loop, 16447 tokens) and every loop's
attention output. The last layer, the chained comparator, the BF16
comparator, the Huginn-shaped workloads (8 loops in one group; 32 loops in
eight anchor groups), the 2-bit loops in groups of 16, the paged cache and
the capacity shape are checked on a sample of (batch, head) series. The oracle works
on its own quantization of the same bf16 inputs; nothing the HIP path writes
is fed to it.
"""
import math
import random

import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (TOL_ATTN, assert_cache_parity, compare_cache, host_copy, log, max_rel_err,
                       oracle_attention, oracle_layer, shuffled_table, u16)
import oracle as O

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS["ouro_16k"]
STEPS = 64
LAST, PREV = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP
CHECK_STEPS = (0, STEPS - 1)


def _sample_units(n, seed, w=W):
    rnd = random.Random(seed)
    units = {(0, 0), (w.batch - 1, w.heads - 1)}
    while len(units) < n:
        units.add((rnd.randrange(w.batch), rnd.randrange(w.heads)))
    return sorted(units)


def _build(layer, policy, bits, w=W, block_size=0):
    """Inputs and a GPU cache holding tokens [0, T + STEPS - 1) of `layer`; block_size > 0
    makes it a paged cache over a shuffled pool."""
    B, H, D, T = w.batch, w.heads, w.D, w.T
    T_max = T + STEPS
    X = synth.kv(w, layer, 0, T_max, device="cuda")
    rk, rv = synth.rotation(w, layer, 0), synth.rotation(w, layer, 1)
    nb, table = shuffled_table(B, T_max, block_size, [T_max] * B, seed=layer) if block_size else (0, None)
    d = rq.make_desc(B, H, D, list(bits), T_max, policy, group=w.groups_for(bits), loop_group=w.loop_group,
                     block_size=block_size, num_blocks=nb)
    cache = rq.LayerCache.allocate(d, rk, rv, block_table=table)
    log(f"layer {layer} policy {policy}: bulk store of {T} tokens")
    rq.quantize_append(cache, X[..., :T, :].contiguous(), torch.zeros(B, dtype=torch.int32, device="cuda"), T)
    for k in range(STEPS - 1):
        pos = torch.full((B,), T + k, dtype=torch.int32, device="cuda")
        rq.quantize_append(cache, X[..., T + k:T + k + 1, :].contiguous(), pos, 1)
    torch.cuda.synchronize()
    return X, rk, rv, cache


def _gpu_outputs(X, cache, layer, w=W):
    """{(step, loop): (out [B][H][D] on the host, q, k_cur, v_cur)} in the benchmark's call order."""
    B, H, D, T = w.batch, w.heads, w.D, w.T
    ws = rq.alloc_workspace(cache.desc)
    res = {}
    for k in CHECK_STEPS:
        past = torch.full((B,), T + k, dtype=torch.int32, device="cuda")
        for r in range(w.L):
            q = synth.query(w, layer, r, k, device="cuda")
            kc = X[0, r, :, :, T + k].contiguous()
            vc = X[1, r, :, :, T + k].contiguous()
            out = torch.empty(B, H, D, device="cuda")
            rq.decode_attn(cache, r, q, kc, vc, past, 1.0 / math.sqrt(D), out, ws)
            res[(k, r)] = (out, q, kc, vc)
    torch.cuda.synchronize()
    return res


def _check(layer, policy, bits, units, label, w=W, block_size=0):
    X, rk, rv, cache = _build(layer, policy, bits, w, block_size)
    outs = _gpu_outputs(X, cache, layer, w)
    Tc = w.T + STEPS - 1
    host = host_copy(cache)
    worst = 0.0
    for i in range(0, len(units), 16):
        chunk = units[i:i + 16]
        log(f"{label}: oracle for units {i}..{i + len(chunk) - 1} of {len(units)}")
        series = oracle_layer(X, rk, rv, bits, policy, Tc, units=chunk, loop_group=w.loop_group,
                              groups=w.groups_for(bits))
        assert_cache_parity(compare_cache(cache, series, Tc, host=host), f"{label} units {i}+")
        for (k, r), (out, q, kc, vc) in outs.items():
            lens = [w.T + k] * w.batch
            ref = oracle_attention(series, chunk, r, lens, rk, rv, q, kc, vc, 1.0 / math.sqrt(w.D))
            err = max_rel_err(out, ref)
            worst = max(worst, err)
            assert err <= TOL_ATTN, (label, k, r, err)
        del series
    log(f"{label}: attention max rel err {worst:.3e} over steps {CHECK_STEPS}, all loops")


def test_ouro_16k_layer0_every_series():
    _check(0, LAST, W.bits, [(b, h) for b in range(W.batch) for h in range(W.heads)], "16k layer 0")


def test_ouro_16k_last_layer_sampled():
    _check(W.layers - 1, LAST, W.bits, _sample_units(8, 23), f"16k layer {W.layers - 1}")


def test_ouro_16k_chained_sampled():
    _check(0, PREV, W.chained_bits, _sample_units(8, 7), "16k chained layer 0")


def test_huginn_4k_sampled():
    """Huginn-shaped workload at full size (B4, H55, D96, 8 loops, 4096 tokens): the
    last layer, sampled series, every loop."""
    w = synth.WORKLOADS["huginn_4k"]
    _check(w.layers - 1, LAST, w.bits, _sample_units(8, 5, w), "huginn 4k", w)


def test_huginn_4k_chained_sampled():
    """The Huginn-shaped workload's chained comparator at full size (one group of 8
    loops, plan [4,4,2,2,2,2,2,2]: decoding loop j reads j stored components, up to
    8): the last layer, sampled series, every loop."""
    w = synth.WORKLOADS["huginn_4k"]
    _check(w.layers - 1, PREV, w.chained_bits, _sample_units(6, 9, w), "huginn 4k chained", w)


@pytest.mark.parametrize("policy", [LAST, PREV])
def test_huginn32_groups_sampled(policy):
    """Huginn-3.5B as the paper groups it (B4, H55, D96, 32 loops in eight anchor
    groups of four, 4096 tokens): layer 0, sampled series, every loop, both the
    shared-anchor and the chained policy."""
    w = synth.WORKLOADS["huginn32_4k"]
    bits = w.bits if policy == LAST else w.chained_bits
    _check(0, policy, bits, _sample_units(6, 13 + policy, w), f"huginn32 G4 policy={policy}", w)


def test_ouro_16k_group16_sampled():
    """The 16k workload with its 2-bit loops in groups of 16 channels: layer 0, sampled
    series, every loop."""
    w = synth.WORKLOADS["ouro_16k_g16"]
    _check(0, LAST, w.bits, _sample_units(8, 17, w), "16k g16", w)


def test_ouro_16k_paged_sampled():
    """The 16k workload in a paged cache (16-token blocks over a shuffled pool, the
    benchmark's paged configuration): layer 0, sampled series, every loop."""
    _check(0, LAST, W.bits, _sample_units(8, 29), "16k paged BS16", W, block_size=16)


def test_capacity_8k_batch64_sampled():
    """Capacity shape (8192 tokens, batch 64): one slot per (batch, head), sampled series."""
    w = synth.WORKLOADS["ouro_8k_capacity"].with_(batch=64)
    _check(0, LAST, w.bits, _sample_units(8, 3, w), "8k B64", w)


def test_ouro_int2_4k_every_series():
    """Uniform-INT2 Ouro shape at its full size (B1, H16, D128, 4 loops, 4096 cached
    tokens, plan [2,2,2,2]; capacity 4096 + 64, so the benchmark's split plan of 16 slots
    per series): layer 0, every (batch, head) series, the whole cache and every loop's
    output at the first and last step."""
    w = synth.WORKLOADS["ouro_int2_4k"]
    d = rq.make_desc(w.batch, w.heads, w.D, list(w.bits), w.T + STEPS)
    unit, nsplit = rq.split_plan(d)
    log(f"int2 4k: {nsplit} slots of {rq.slot_len(w.T, nsplit, unit)} tokens per series")
    _check(0, LAST, w.bits, [(b, h) for b in range(w.batch) for h in range(w.heads)], "int2 4k layer 0", w)


def test_ouro_16k_bf16_sampled():
    B, H, D, T = W.batch, W.heads, W.D, W.T
    layer = 0
    X = synth.kv(W, layer, 0, T + STEPS, device="cuda")
    d = rq.make_desc(B, H, D, list(W.bits), T + STEPS)
    ws = rq.alloc_workspace(d)
    units = _sample_units(8, 11)
    worst = 0.0
    for k in CHECK_STEPS:
        past = torch.full((B,), T + k, dtype=torch.int32, device="cuda")
        for r in range(W.L):
            q = synth.query(W, layer, r, k, device="cuda")
            kc = X[0, r, :, :, T + k].contiguous()
            vc = X[1, r, :, :, T + k].contiguous()
            out = torch.empty(B, H, D, device="cuda")
            log(f"16k bf16 step {k} loop {r}")
            rq.decode_attn_bf16(d, X[0, r], X[1, r], q, kc, vc, past, 1.0 / math.sqrt(D), out, ws)
            torch.cuda.synchronize()
            qn, kn, vn = u16(q), u16(kc), u16(vc)
            ref = {}
            for b, h in units:
                Kh = u16(X[0, r, b, h, :T + k])
                Vh = u16(X[1, r, b, h, :T + k])
                ref[(b, h)] = O.attend_bf16(Kh, Vh, qn[b, h], kn[b, h], vn[b, h], 1.0 / math.sqrt(D))
            err = max_rel_err(out, ref)
            worst = max(worst, err)
            assert err <= TOL_ATTN
    log(f"16k bf16: max rel err {worst:.3e}")


def test_long_context_many_slots():
    """One sequence of 65536 cached tokens over two heads (D128, plan [2,2,4,4]): the
    split plan gives 256 slots of 8 tiles per (b, h), so every launch streams short
    slots and the combine merges 256 partials in sixteen rounds of loads. Both
    series, the whole cache and every loop's output at the first and last step."""
    w = W.with_(batch=1, heads=2, T=65536, layers=1)
    d = rq.make_desc(w.batch, w.heads, w.D, list(w.bits), w.T + STEPS)
    unit, nsplit = rq.split_plan(d)
    log(f"64k B1 H2: {nsplit} slots of {rq.slot_len(w.T, nsplit, unit)} tokens")
    assert nsplit >= 64
    _check(0, LAST, w.bits, [(0, 0), (0, 1)], "64k B1 H2", w)
