"""Rotations stored in fp16 (RQ_FLAG_ROT_F16).

The paper keeps its learned per-head rotations in FP16 once calibrated and
multiplies them with FP16 inputs and FP32 accumulation (App. G). Every kernel
here converts fp16 entries to fp32/fp64 exactly and keeps its arithmetic, so
a cache stored and decoded with fp16 matrices must hold exactly the bytes, and
give exactly the outputs, of the same matrices held in fp32. That is checked
for the one-token and bulk appends, the layered append, every decode variant
(contiguous, paged, chains of up to eight components, the 21-bit query, the
no-workspace entry point, partial + combine) at head dims 64, 96 and 128; one
shape is also compared with the oracle given the fp16 matrices.
"""
import math

import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, inputs, log,
                       oracle_layer, shuffled_table)

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP
F16 = rq.FLAG_ROT_F16

# label, workload, D, bits, policy, loop_group, groups, block size (0: contiguous)
CASES = [
    ("last-d128", "tiny", 128, (2, 2, 4, 4), LAST, 0, 32, 0),
    ("first-g16-d64", "tiny", 64, (4, 2, 2, 2), FIRST, 0, [32, 16, 16, 16], 0),
    ("prev-chain8-d96", "huginn_4k", 96, (4, 4, 2, 2, 2, 2, 2, 2), PREV, 0, 32, 0),
    ("last-groups-d96", "huginn_4k", 96, (2, 2, 2, 4, 2, 2, 2, 4), LAST, 4, 32, 0),
    ("prev-paged-d128", "tiny", 128, (4, 4, 2, 2), PREV, 0, 32, 16),
]


def buffers(c: rq.LayerCache):
    L = c.desc.loops
    out = [c.codes[kv][r] for kv in range(2) for r in range(L)]
    out += [c.meta[kv][r] for kv in range(2) for r in range(L)]
    out += [c.alpha[kv][r] for kv in range(2) for r in range(L) if c.alpha[kv][r] is not None]
    return out


def fp16_pair(rk, rv):
    """The rotations rounded to fp16, and the same values held in fp32."""
    rk16, rv16 = rk.half(), rv.half()
    return rk16, rv16, rk16.float(), rv16.float()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp16_rotations_equal_fp32_copy(case):
    label, wname, D, bits, policy, lg, groups, bs = case
    B, H, T = 3, 2, 304
    w = synth.WORKLOADS[wname].with_(batch=B, heads=H, D=D, L=len(bits), bits=tuple(bits),
                                     chained_bits=tuple(bits), loop_group=lg)
    X, rk, rv = inputs(w, T + 1, batch=B)
    rk16, rv16, rk32, rv32 = fp16_pair(rk, rv)
    lens = [T, 97, 0]
    paging = None
    if bs:
        nb, table = shuffled_table(B, T + 16, bs, [T + 16] * B, seed=3)
        paging = (bs, nb, table)
    T_max = T + 16
    caches = []
    for r16, flags in (((rk16, rv16), F16), ((rk32, rv32), 0)):
        log(f"{label}: build flags={flags}")
        # a bulk append, then appends of 3 tokens and of single tokens (the per-unit kernel)
        caches.append(build_gpu_layer(X, r16[0], r16[1], bits, policy, T_max=T_max, T=T, steps_of_one=40,
                                      chunk=3, loop_group=lg, groups=groups, paging=paging, flags=flags,
                                      zero=True))
    c16, c32 = caches
    assert c16.rot[0].dtype == torch.float16 and c32.rot[0].dtype == torch.float32
    for i, (x, y) in enumerate(zip(buffers(c16), buffers(c32))):
        assert torch.equal(x, y), (label, "buffer", i)

    d16, d32 = c16.desc, c32.desc
    ws16, ws32 = rq.alloc_workspace(d16), rq.alloc_workspace(d32)
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    decoded = 0
    for r in range(len(bits)):
        if rq.check_decode(d16, r) != 0:
            continue
        decoded += 1
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        for flags in (None, rq.FLAG_PRECISE_QUERY):
            o16 = torch.empty(B, H, D, dtype=torch.float32, device="cuda")
            o32 = torch.empty_like(o16)
            rq.decode_attn(c16, r, q, kc, vc, past, scale, o16, ws16, flags=flags)
            rq.decode_attn(c32, r, q, kc, vc, past, scale, o32, ws32, flags=flags)
            torch.cuda.synchronize()
            assert torch.isfinite(o16).all()
            assert torch.equal(o16, o32), (label, r, flags)
            if flags is None:
                o_default = o16
        # no-workspace entry point and the two launches called separately
        on = torch.empty(B, H, D, dtype=torch.float32, device="cuda")
        rq.decode_attn_noalloc(c16, r, q, kc, vc, past, scale, on)
        op = torch.empty_like(on)
        rq.decode_attn_partial(c16, r, q, past, scale, ws16)
        rq.decode_combine(d16, c16.rot[1], q, kc, vc, past, scale, op, ws16)
        torch.cuda.synchronize()
        assert torch.equal(on, o_default) and torch.equal(op, o_default), (label, r)
    assert decoded > 0
    log(f"{label}: caches and {decoded} loops' outputs bit-identical")


def test_fp16_rotations_layered_append():
    """rq_quantize_append_layers with fp16 rotations writes the bytes of the fp32 copies."""
    B, H, D, T_max, nl = 3, 2, 96, 64, 5
    bits = (4, 2, 2, 2)
    stacks = []
    g = torch.Generator(device="cuda").manual_seed(2)
    kv = (3.0 * torch.randn(nl, 2, len(bits), B, H, 1, D, generator=g, device="cuda")).to(torch.bfloat16)
    pos = torch.tensor([5, 0, T_max - 1], dtype=torch.int32, device="cuda")
    w = synth.WORKLOADS["huginn_4k"].with_(heads=H)
    for flags in (F16, 0):
        d = rq.make_desc(B, H, D, bits, T_max, LAST, flags=flags)
        caches = []
        for l in range(nl):
            rk16, rv16, rk32, rv32 = fp16_pair(synth.rotation(w, l, 0), synth.rotation(w, l, 1))
            c = rq.LayerCache.allocate(d, *((rk16, rv16) if flags else (rk32, rv32)))
            for x in buffers(c):
                x.zero_()
            caches.append(c)
        rq.quantize_append_layers(caches, kv, pos, 1)
        stacks.append(caches)
    torch.cuda.synchronize()
    for l in range(nl):
        for i, (x, y) in enumerate(zip(buffers(stacks[0][l]), buffers(stacks[1][l]))):
            assert torch.equal(x, y), (l, i)


def test_fp16_rotations_against_oracle():
    """The oracle given the fp16 matrices (exact in its fp32 input): cache and attention parity."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=3, D=128, nb=128, outliers=4)
    T = 520
    X, rk, rv = inputs(w, T + 1, batch=2)
    rk16, rv16 = rk.half(), rv.half()
    bits = (2, 2, 4, 4)
    cache = build_gpu_layer(X, rk16, rv16, bits, LAST, T_max=T + 1, T=T, steps_of_one=5, flags=F16)
    series = oracle_layer(X, rk16, rv16, bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), "fp16 rotations")
    decode_and_compare(w, X, rk16, rv16, cache, series, [T, 131], range(4), "fp16 rotations")
