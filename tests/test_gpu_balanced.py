"""GPU parity of the fused decode call's balanced partition (rq_decode_attn where
nsplit equal slots per (b, h) would load the compute units unevenly).

Shapes of B H = 300 series: the slot plan gives 300 workgroups on 256 compute
units, so the call cuts the tiles of all series into equal chunks instead, one
per workgroup, and a series' pieces span several workgroups. Ragged lengths
(empty sequences, one token, tile edges) make pieces start and end inside
sequences and skip empty ones. Outputs are compared with the oracle for every
(b, h) and loop, with the documented slot path (partial + combine, another
merge order), and with the call without a workspace (the same kernels).
"""
import math

import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (TOL_ATTN, assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare,
                       inputs, log, oracle_layer)

pytestmark = pytest.mark.gpu

LAST = rq.POLICY_LAST_LOOP

CASES = [
    # workload, D, batch, heads, bits, cached tokens, per-sequence lengths
    ("huginn_4k", 96, 5, 60, None, 700, [0, 1, 43, 377, 699]),
    ("tiny", 128, 2, 150, (2, 2, 4, 4), 500, [500, 31]),
    ("tiny", 64, 3, 100, (2, 2, 4, 4), 600, [600, 0, 250]),
]


@pytest.mark.parametrize("wname,D,B,H,bits,T,lens", CASES, ids=["d96-8loops", "d128", "d64"])
def test_balanced_decode(wname, D, B, H, bits, T, lens):
    w = synth.WORKLOADS[wname].with_(batch=B, heads=H, D=D, nb=min(D, 128)) if wname == "tiny" else \
        synth.WORKLOADS[wname].with_(batch=B, heads=H)
    bits = tuple(bits or w.bits)
    label = f"balanced D{D} B{B} H{H}"
    log(label)
    X, rk, rv = inputs(w, T + 1, batch=B)
    cache = build_gpu_layer(X, rk, rv, bits, LAST, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, bits, LAST, T)
    assert_cache_parity(compare_cache(cache, series, T), label + " cache")
    d = cache.desc
    unit, nsplit = rq.split_plan(d)
    slot_bytes = B * H * nsplit * (D + 4) * 4
    log(f"{label}: {nsplit} slot(s) of {unit}-token tiles per series; workspace {rq.workspace_bytes(d)} "
        f"bytes against {slot_bytes} for the slots")
    # the balanced partition keeps more partial rows per series than the slots
    assert rq.workspace_bytes(d) > slot_bytes
    decode_and_compare(w, X, rk, rv, cache, series, lens, range(len(bits)), label, batch=B)

    # the documented slots (partial + combine) and the no-workspace call
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    ws_a, ws_b = rq.alloc_workspace(d), rq.alloc_workspace(d)
    for r in (0, len(bits) - 1):
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        fused, slots, noalloc = (torch.empty(B, H, D, device="cuda") for _ in range(3))
        log(f"{label}: fused, slots and no-workspace calls, loop {r}")
        rq.decode_attn(cache, r, q, kc, vc, past, scale, fused, ws_a)
        rq.decode_attn_partial(cache, r, q, past, scale, ws_b)
        rq.decode_combine(d, cache.rot[1], q, kc, vc, past, scale, slots, ws_b)
        rq.decode_attn_noalloc(cache, r, q, kc, vc, past, scale, noalloc)
        torch.cuda.synchronize()
        assert torch.equal(fused, noalloc)
        rel = ((fused - slots).abs().max() / slots.abs().max()).item()
        log(f"{label}: loop {r} balanced vs slots max rel diff {rel:.3e}")
        assert rel <= 1e-5, rel
        assert rel <= TOL_ATTN
