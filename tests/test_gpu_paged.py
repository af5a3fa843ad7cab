"""GPU parity of the paged cache (block table; paper §4.2: the compressed cache
lives in the serving engine's paged KV blocks).

A paged cache must hold, token for token, what a contiguous cache holds, and
decode over it must give the contiguous call's output bit for bit: the kernels
differ only in where a token's row is. Block tables scatter every sequence
over a shuffled pool with unused blocks; entries past a sequence's tokens are
-1 and must never be read. The caches and outputs are also compared with the
oracle.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, host_copy, inputs,
                       log, oracle_layer, shuffled_table)

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP


def _pair(w, bits, policy, T, T_max, BS, lens_alloc, steps_of_one, chunk, groups=32, seed=0):
    """The same tokens stored in a contiguous and in a paged cache."""
    B = w.batch
    X, rk, rv = inputs(w, T_max, batch=B)
    nb, table = shuffled_table(B, T_max, BS, lens_alloc, seed=seed)
    common = dict(steps_of_one=steps_of_one, chunk=chunk, loop_group=w.loop_group, groups=groups)
    flat = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, **common)
    paged = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, paging=(BS, nb, table), **common)
    return X, rk, rv, flat, paged


def _same_cache(flat, paged, T):
    hf, hp = host_copy(flat), host_copy(paged)
    for key, (cf, mf, af) in hf.items():
        cp, mp, ap = hp[key]
        assert np.array_equal(cf[:, :, :T], cp[:, :, :T]), key
        assert np.array_equal(mf[:, :, :T], mp[:, :, :T]), key
        if af is not None:
            assert np.array_equal(af[:, :, :T], ap[:, :, :T]), key


def _same_outputs(w, X, flat, paged, lens, loops):
    B, H, D = X.shape[2], X.shape[3], X.shape[5]
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws1, ws2 = rq.alloc_workspace(flat.desc), rq.alloc_workspace(paged.desc)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r in loops:
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        o1 = torch.empty(B, H, D, device="cuda")
        o2 = torch.empty(B, H, D, device="cuda")
        rq.decode_attn(flat, r, q, kc, vc, past, 1.0 / math.sqrt(D), o1, ws1)
        rq.decode_attn(paged, r, q, kc, vc, past, 1.0 / math.sqrt(D), o2, ws2, dev_err=err)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), (r, (o1 - o2).abs().max().item())
    assert int(err.item()) == 0


@pytest.mark.parametrize("D,BS,policy,bits", [
    (64, 16, LAST, (2, 2, 2, 4)),
    (128, 64, LAST, (2, 2, 4, 4)),
    (96, 16, PREV, (4, 4, 2, 2)),
    (128, 256, FIRST, (4, 2, 2, 2)),
])
def test_paged_equals_contiguous_and_oracle(D, BS, policy, bits):
    """Bulk and few-token appends (crossing block edges), ragged decode lengths."""
    w = synth.WORKLOADS["tiny"].with_(batch=3, heads=2, D=D, nb=32 if D == 96 else 0, outliers=4)
    T, T_max = 700, 1024
    lens = [T, 0, 333]
    X, rk, rv, flat, paged = _pair(w, bits, policy, T, T_max, BS, [T + 1] * 3, steps_of_one=37, chunk=5)
    label = f"paged D{D} BS{BS} policy={policy}"
    log(label)
    _same_cache(flat, paged, T)
    _same_outputs(w, X, flat, paged, lens, range(4))
    series = oracle_layer(X, rk, rv, bits, policy, T)
    assert_cache_parity(compare_cache(paged, series, T), label)
    decode_and_compare(w, X, rk, rv, paged, series, lens, range(4), label)


def test_paged_groups_of_16_and_loop_groups():
    w = synth.WORKLOADS["huginn_4k"].with_(batch=2, heads=2, loop_group=4)
    bits = (2, 2, 2, 4) * 2
    groups = [16 if b == 2 else 32 for b in bits]
    T, T_max = 300, 512
    X, rk, rv, flat, paged = _pair(w, bits, LAST, T, T_max, 32, [T + 1] * 2, steps_of_one=4, chunk=1,
                                   groups=groups, seed=3)
    _same_cache(flat, paged, T)
    _same_outputs(w, X, flat, paged, [T, 100], range(8))


def test_paged_32_loops():
    """32 loops: every append takes the per-unit kernel."""
    w = synth.WORKLOADS["huginn32_4k"].with_(batch=2, heads=1)
    T, T_max = 90, 128
    X, rk, rv, flat, paged = _pair(w, w.bits, LAST, T, T_max, 16, [T + 1] * 2, steps_of_one=3, chunk=1, seed=5)
    _same_cache(flat, paged, T)
    _same_outputs(w, X, flat, paged, [T, 17], (0, 3, 30, 31))


@pytest.mark.parametrize("BS", [16, 64])
def test_paged_unused_entries_are_never_read(BS):
    """Each sequence's table stops at its own length (-1 past it): appends and decode of
    shorter sequences touch no entry beyond, and flag nothing. D128: blocks of 16 take
    the lane-by-lane kernel, blocks of 64 the one-block-per-tile kernel."""
    w = synth.WORKLOADS["tiny"].with_(batch=3, heads=2, D=128)
    T_max = 512
    lens = [200, 37, 0]
    B, H, D = 3, 2, 128
    X, rk, rv = inputs(w, T_max, batch=B)
    nb, table = shuffled_table(B, T_max, BS, [n + 1 for n in lens], seed=7)
    d = rq.make_desc(B, H, D, w.bits, T_max, LAST, block_size=BS, num_blocks=nb)
    cache = rq.LayerCache.allocate(d, rk, rv, block_table=table)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # one sequence at a time through the few-token path: B appends of its own length
    for b, n in enumerate(lens):
        for t0 in range(0, n, 8):
            k = min(8, n - t0)
            pos = torch.full((B,), -10**6, dtype=torch.int32, device="cuda")
            pos[b] = t0                      # the other sequences' tokens fall before 0: dropped
            rq.quantize_append(cache, X[..., t0:t0 + k, :].contiguous(), pos, k, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == rq.DEVERR_CAPACITY     # only the deliberately dropped positions
    err.zero_()
    flat = build_gpu_layer(X, rk, rv, w.bits, LAST, T_max=T_max, T=max(lens))
    hf, hp = host_copy(flat), host_copy(cache)
    for key in hf:
        for b, n in enumerate(lens):
            assert np.array_equal(hf[key][0][b, :, :n], hp[key][0][b, :, :n]), (key, b)
    _same_outputs(w, X, flat, cache, lens, range(4))


@pytest.mark.parametrize("D,BS", [(64, 16), (128, 32)])
def test_paged_invalid_block_flags_and_reads_zero(D, BS):
    """A table entry outside [0, num_blocks) in the used range: append drops those tokens
    and decode reads them as zeros, both flag RQ_DEVERR_BLOCK; nothing else changes."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=D)
    T_max, T = 256, 100
    B, H = 2, 2
    X, rk, rv = inputs(w, T_max, batch=B)
    nb, table = shuffled_table(B, T_max, BS, [T + 1, T + 1], seed=11)
    table[1, 1] = nb                       # one block of sequence 1 points past the pool
    d = rq.make_desc(B, H, D, w.bits, T_max, LAST, block_size=BS, num_blocks=nb)
    cache = rq.LayerCache.allocate(d, rk, rv, block_table=table)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rq.quantize_append(cache, X[..., :T, :].contiguous(), torch.zeros(B, dtype=torch.int32, device="cuda"), T,
                       dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == rq.DEVERR_BLOCK
    err.zero_()
    ws = rq.alloc_workspace(d)
    past = torch.tensor([T, T], dtype=torch.int32, device="cuda")
    q = synth.query(w, 0, 0, 0, device="cuda", batch=B)
    kc = X[0, 0, :, :, T].contiguous()
    vc = X[1, 0, :, :, T].contiguous()
    out = torch.empty(B, H, D, device="cuda")
    rq.decode_attn(cache, 0, q, kc, vc, past, 0.125, out, ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == rq.DEVERR_BLOCK
    assert torch.isfinite(out).all()
    # sequence 0 is untouched by the bad entry: same as a contiguous cache
    flat = build_gpu_layer(X, rk, rv, w.bits, LAST, T_max=T_max, T=T)
    o2 = torch.empty(B, H, D, device="cuda")
    rq.decode_attn(flat, 0, q, kc, vc, past, 0.125, o2, rq.alloc_workspace(flat.desc))
    torch.cuda.synchronize()
    assert torch.equal(out[0], o2[0])
