"""rq_decode_attn_noalloc (the decode call that allocates nothing: its split
partials live in the library's static per-device scratch) against
rq_decode_attn with a caller workspace, through the C ABI: bit-identical outputs
on two calls in a row, the second one smaller, and a request larger than the
scratch rejected on the host."""
import ctypes
import math

import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import build_gpu_layer, log

pytestmark = pytest.mark.gpu


def _case(B, H, D, T, bits, policy, seed):
    w = synth.WORKLOADS["tiny"].with_(batch=B, heads=H, D=D, nb=32 if D == 96 else D, seed=seed)
    X = synth.kv(w, 0, 0, T + 1, device="cuda", batch=B)
    rk, rv = synth.rotation(w, 0, 0), synth.rotation(w, 0, 1)
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T)
    return w, X, cache


def _compare(w, X, cache, lens, label):
    d = cache.desc
    B, H, D = d.batch, d.heads, d.head_dim
    ws = rq.alloc_workspace(d)
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    for r in range(d.loops):
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        ref = torch.empty(B, H, D, device="cuda")
        got = torch.full((B, H, D), float("nan"), device="cuda")
        rq.decode_attn(cache, r, q, kc, vc, past, scale, ref, ws)
        rq.decode_attn_noalloc(cache, r, q, kc, vc, past, scale, got)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), (label, r, (ref - got).abs().max().item())
    log(f"{label}: no-alloc decode equals the workspace decode on every loop")


def test_noalloc_equals_workspace_decode_two_calls():
    """A larger call, then a smaller one (fewer series, tokens and slots) on the same
    device: both equal the workspace path bit for bit, so nothing of the first call's
    scratch contents leaks into the second."""
    big = _case(3, 4, 128, 700, (2, 2, 4, 4), rq.POLICY_LAST_LOOP, seed=1)
    assert rq.workspace_bytes(big[2].desc) <= rq.SCRATCH_BYTES
    _compare(*big, lens=[700, 0, 333], label="no-alloc B3 H4 D128")
    small = _case(1, 2, 96, 100, (4, 2, 2, 2), rq.POLICY_PREV_LOOP, seed=2)
    assert rq.workspace_bytes(small[2].desc) < rq.workspace_bytes(big[2].desc)
    _compare(*small, lens=[57], label="no-alloc B1 H2 D96 chained")


def test_noalloc_rejects_requests_beyond_the_scratch():
    """B*H*nsplit partials beyond RQ_SCRATCH_BYTES: RQ_E_SCRATCH, nothing enqueued."""
    d = rq.make_desc(128, 128, 128, [2, 2, 4, 4], 256)
    assert rq.workspace_bytes(d) > rq.SCRATCH_BYTES
    c = rq.LayerCacheC()
    for kv in range(2):
        for r in range(4):
            c.codes[kv][r] = c.meta[kv][r] = c.alpha[kv][r] = 0x100000
        c.rot[kv] = 0x100000
    fake = ctypes.c_void_p(0x100000)
    code = rq.lib.rq_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(c), 0, fake, fake, fake, fake,
                                         ctypes.c_float(0.1), fake, None, 0)
    assert code == 11 and rq.STATUS[code] == "RQ_E_SCRATCH"
