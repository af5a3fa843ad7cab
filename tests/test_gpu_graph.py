"""Decode steps captured in a HIP graph and replayed, as the benchmark runs them.

Device-resident lengths make a step capturable: every replay must reproduce the
eager step bit for bit, with eager work and synchronizations between the
replays (contiguous and paged caches).
"""
import math

import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import build_gpu_layer, inputs, log, shuffled_table

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("paged", [False, True])
def test_graph_replays_match_eager(paged):
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=128, outliers=4)
    B, H, D, L = w.batch, w.heads, w.D, w.L
    T, T_max = 300, 320
    X, rk, rv = inputs(w, T_max, batch=B)
    paging = None
    if paged:
        nb, table = shuffled_table(B, T_max, 32, [T_max] * B, seed=2)
        paging = (32, nb, table)
    cache = build_gpu_layer(X, rk, rv, w.bits, rq.POLICY_LAST_LOOP, T_max=T_max, T=T, paging=paging)
    ws = rq.alloc_workspace(cache.desc)
    past = torch.full((B,), T, dtype=torch.int32, device="cuda")
    qs = [synth.query(w, 0, r, 0, device="cuda", batch=B) for r in range(L)]
    kv_cur = X[..., T:T + 1, :].contiguous()                       # [2][L][B][H][1][D]
    outs = torch.empty(L, B, H, D, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def step():
        for r in range(L):
            rq.decode_attn(cache, r, qs[r], kv_cur[0, r, :, :, 0].contiguous(), kv_cur[1, r, :, :, 0].contiguous(),
                           past, scale, outs[r], ws)
        rq.quantize_append(cache, kv_cur, past, 1)
        past.add_(1)

    step()                                                         # eager
    torch.cuda.synchronize()
    ref = outs.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    past.fill_(T)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        past.fill_(T)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref), f"replay {i} differs from the eager step"
        assert int(past[0].item()) == T + 1
        # eager work between replays: a decode of another length
        past.fill_(T - 7)
        tmp = torch.empty(B, H, D, device="cuda")
        rq.decode_attn(cache, 1, qs[1], kv_cur[0, 1, :, :, 0].contiguous(), kv_cur[1, 1, :, :, 0].contiguous(), past,
                       scale, tmp, ws)
        torch.cuda.synchronize()
    log(f"graph replays ({'paged' if paged else 'contiguous'}): 4 of 4 equal to the eager step")


@pytest.mark.parametrize("paged", [False, True])
def test_graph_replays_layered_append(paged):
    """Two layers' decode calls and one rq_quantize_append_layers call captured as a
    step: every replay reproduces the eager step's outputs and cache bytes."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=128, outliers=4)
    B, H, D, L = w.batch, w.heads, w.D, w.L
    T, T_max, NL = 200, 256, 2
    paging = None
    if paged:
        nb, table = shuffled_table(B, T_max, 64, [T_max] * B, seed=3)
        paging = (64, nb, table)
    caches, kvs = [], []
    for l in range(NL):
        X, rk, rv = inputs(w, T_max, layer=l, batch=B)
        caches.append(build_gpu_layer(X, rk, rv, w.bits, rq.POLICY_LAST_LOOP, T_max=T_max, T=T, paging=paging))
        kvs.append(X[..., T:T + 1, :])
    kv_cur = torch.stack(kvs).contiguous()                        # [NL][2][L][B][H][1][D]
    ws = rq.alloc_workspace(caches[0].desc)
    past = torch.full((B,), T, dtype=torch.int32, device="cuda")
    qs = [synth.query(w, l, r, 0, device="cuda", batch=B) for l in range(NL) for r in range(L)]
    outs = torch.empty(NL, L, B, H, D, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def step():
        for r in range(L):
            for l in range(NL):
                rq.decode_attn(caches[l], r, qs[l * L + r], kv_cur[l, 0, r, :, :, 0].contiguous(),
                               kv_cur[l, 1, r, :, :, 0].contiguous(), past, scale, outs[l, r], ws)
        rq.quantize_append_layers(caches, kv_cur, past, 1)
        past.add_(1)

    bufs = [t for c in caches for kv in range(2) for t in c.codes[kv] + c.meta[kv] + c.alpha[kv] if t is not None]

    def row_bytes():
        torch.cuda.synchronize()
        return [t.clone() for t in bufs]

    def poison_row_T():
        """Overwrite every buffer's row of position T (the decode reads only rows < T)."""
        for t in bufs:
            junk = 0xA5 if t.dtype == torch.uint8 else -23131          # bytes 0xA5
            if paged:
                tb = paging[2].cpu()
                for b in range(B):
                    t[int(tb[b, T // 64]), :, T % 64] = junk
            else:
                t[:, :, T] = junk

    step()                                                         # eager
    torch.cuda.synchronize()
    ref_out, ref_cache = outs.clone(), row_bytes()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    past.fill_(T)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        past.fill_(T)
        outs.zero_()
        poison_row_T()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_out), f"replay {i}: outputs differ from the eager step"
        assert all(torch.equal(a, b) for a, b in zip(row_bytes(), ref_cache)), f"replay {i}: cache differs"
        assert int(past[0].item()) == T + 1
        # eager work between replays: a decode of another length
        past.fill_(T - 5)
        tmp = torch.empty(B, H, D, device="cuda")
        rq.decode_attn(caches[1], 0, qs[L], kv_cur[1, 0, 0, :, :, 0].contiguous(), kv_cur[1, 1, 0, :, :, 0].contiguous(),
                       past, scale, tmp, ws)
        torch.cuda.synchronize()
    log(f"graph replays with the layered append ({'paged' if paged else 'contiguous'}): 4 of 4 equal to the eager step")
