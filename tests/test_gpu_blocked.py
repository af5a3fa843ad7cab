"""GPU parity of the blocked cache layout (rq.h, rq_layer_cache.block_bytes):
each loop's K and V codes, metadata and alpha share blocks of 32 token rows.

The layout changes only where the kernels read and write a token's row, so a
blocked cache must hold exactly what the separate-buffer cache holds, value for
value, after bulk and few-token appends, and every decode over it must give
the separate cache's output bit for bit: contiguous and paged caches, Last-,
First- and Previous-loop plans (chains of up to eight components), groups of
16, all three head sizes (64 and 128 take the kernel's fixed-offset path, 96
the per-row one), ragged lengths, and rows past the decoded lengths filled
with NaN patterns (they are read and must be masked). One case is also checked
against the oracle directly.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, host_copy, inputs, log,
                       oracle_layer, shuffled_table)

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP


def _same_cache(a, b, T):
    ha, hb = host_copy(a), host_copy(b)
    for key, (ca, ma, aa) in ha.items():
        cb, mb, ab = hb[key]
        assert np.array_equal(ca[:, :, :T], cb[:, :, :T]), key
        assert np.array_equal(ma[:, :, :T], mb[:, :, :T]), key
        if aa is not None:
            assert np.array_equal(aa[:, :, :T], ab[:, :, :T]), key


def _same_outputs(w, X, a, b, lens, loops, flags=None):
    B, H, D = X.shape[2], X.shape[3], X.shape[5]
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    wa, wb = rq.alloc_workspace(a.desc), rq.alloc_workspace(b.desc)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for r in loops:
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, i, :, lens[i]] for i in range(B)]).contiguous()
        vc = torch.stack([X[1, r, i, :, lens[i]] for i in range(B)]).contiguous()
        o1 = torch.empty(B, H, D, device="cuda")
        o2 = torch.empty(B, H, D, device="cuda")
        rq.decode_attn(a, r, q, kc, vc, past, 1.0 / math.sqrt(D), o1, wa, flags=flags)
        rq.decode_attn(b, r, q, kc, vc, past, 1.0 / math.sqrt(D), o2, wb, dev_err=err, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), (r, (o1 - o2).abs().max().item())
    assert int(err.item()) == 0


@pytest.mark.parametrize("D,policy,bits,groups,G", [
    (128, LAST, (2, 2, 4, 4), 32, 0),
    (96, LAST, (2, 2, 2, 2, 2, 2, 4, 4), 32, 0),
    (64, FIRST, (4, 2, 2, 2), (32, 16, 16, 16), 0),
    (128, PREV, (4, 4, 2, 2), (32, 32, 16, 16), 0),
    (96, PREV, (4, 2, 2, 2, 2, 2, 2, 2), 32, 0),
    (128, LAST, (2, 2, 2, 4, 2, 2, 2, 4), 32, 4),
])
def test_blocked_equals_separate_contiguous(D, policy, bits, groups, G):
    """Bulk append then few-token appends; every loop decoded at ragged lengths."""
    w = synth.WORKLOADS["tiny"].with_(batch=3, heads=2, D=D, nb=32 if D == 96 else 0, outliers=4, L=len(bits),
                                      loop_group=G)
    T, T_max = 520, 640
    lens = [T, 1, 257]
    X, rk, rv = inputs(w, T_max, batch=3)
    common = dict(steps_of_one=21, chunk=4, loop_group=G, groups=groups)
    label = f"blocked D{D} policy={policy} bits={bits} groups={groups} G={G}"
    log(label)
    sep = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, **common)
    blk = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, blocked=True, **common)
    _same_cache(sep, blk, T)
    _same_outputs(w, X, sep, blk, lens, range(len(bits)))
    # rows past every decoded length hold NaN fp16 patterns: masked, outputs unchanged
    jb, jp = divmod(T, rq.ROW_BLOCK)                 # views [B][H][T_max / 32][32][...]
    for r in range(len(bits)):
        for kv in range(2):
            for name in ("meta", "alpha"):
                t = getattr(blk, name)[kv][r]
                if t is not None:
                    t[:, :, jb, jp:].fill_(0x7e00)
                    t[:, :, jb + 1:].fill_(0x7e00)
    torch.cuda.synchronize()
    _same_outputs(w, X, sep, blk, lens, range(len(bits)))
    if D == 128 and policy == LAST:
        _same_outputs(w, X, sep, blk, lens, [0], flags=rq.FLAG_PRECISE_QUERY)


@pytest.mark.parametrize("D,BS,policy,bits", [
    (128, 32, LAST, (2, 2, 4, 4)),
    (96, 64, PREV, (4, 4, 2, 2)),
    (64, 256, FIRST, (4, 2, 2, 2)),
])
def test_blocked_equals_separate_paged(D, BS, policy, bits):
    """Paged caches over a shuffled pool, appends crossing block edges."""
    w = synth.WORKLOADS["tiny"].with_(batch=3, heads=2, D=D, nb=32 if D == 96 else 0, outliers=4)
    T, T_max = 700, 1024
    lens = [T, 0, 333]
    X, rk, rv = inputs(w, T_max, batch=3)
    nb, table = shuffled_table(3, T_max, BS, [T + 1] * 3)
    common = dict(steps_of_one=37, chunk=5, paging=(BS, nb, table))
    log(f"blocked paged D{D} BS{BS} policy={policy}")
    sep = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, **common)
    blk = build_gpu_layer(X, rk, rv, bits, policy, T_max=T_max, T=T, blocked=True, **common)
    _same_cache(sep, blk, T)
    _same_outputs(w, X, sep, blk, lens, range(len(bits)))


def test_blocked_oracle():
    """The blocked cache against the oracle directly: stored values and attention."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=128, outliers=4)
    bits, T, T_max = (2, 2, 4, 4), 300, 384
    X, rk, rv = inputs(w, T_max, batch=2)
    log("blocked oracle D128 [2,2,4,4]")
    cache = build_gpu_layer(X, rk, rv, bits, LAST, T_max=T_max, T=T, steps_of_one=9, chunk=3, blocked=True)
    series = oracle_layer(X, rk, rv, bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "blocked oracle")
    decode_and_compare(w, X, rk, rv, cache, series, [T, 123], range(4), "blocked oracle", batch=2)


def test_blocked_layer_append_and_mixed_calls():
    """The multi-layer append with blocked caches matches one-layer appends, and a
    multi-layer call must not mix blocked and separate caches."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=64)
    bits, T, T_max = (2, 2, 2, 4), 40, 64
    X, rk, rv = inputs(w, T_max, batch=2)
    d = rq.make_desc(2, 2, 64, bits, T_max)
    many = [rq.LayerCache.allocate(d, rk, rv, blocked=True) for _ in range(3)]
    one = [rq.LayerCache.allocate(d, rk, rv, blocked=True) for _ in range(3)]
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    for t in range(T):
        kv = torch.stack([X[..., t:t + 1, :]] * 3).contiguous()
        p = torch.full((2,), t, dtype=torch.int32, device="cuda")
        rq.quantize_append_layers(many, kv, p, 1)
        for c in one:
            rq.quantize_append(c, X[..., t:t + 1, :].contiguous(), p, 1)
    torch.cuda.synchronize()
    for a, b in zip(many, one):
        _same_cache(a, b, T)
    mixed = [rq.LayerCache.allocate(d, rk, rv, blocked=True), rq.LayerCache.allocate(d, rk, rv)]
    with pytest.raises(rq.RQError):
        rq.quantize_append_layers(mixed, torch.stack([X[..., :1, :]] * 2).contiguous(), pos, 1)
