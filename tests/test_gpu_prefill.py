"""GPU parity of the prefill path (paper §4.2 "Prefill": each loop attends
causally over its own BF16 prompt K/V; after the final loop the prompt is
quantized into the cache) against the oracle.

Attention rows are compared one by one: max over rows of
|o_i - ref_i|_inf / |ref_i|_inf, bar 2e-3. The full-size prompt is checked on
sampled rows through the decode oracle, which gives row i of a prefill
exactly (the oracle pins show it).
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_quantize_amd as rq
import oracle as O
import synth
from rq_parity import TOL_ATTN, assert_cache_parity, build_gpu_layer, compare_cache, log, oracle_layer, u16

pytestmark = pytest.mark.gpu


def _qkv(w, n, loop=0, layer=0):
    """bf16 [B][H][n][D] prompt q, k, v of one loop (synthetic queries per position)."""
    X = synth.kv(w, layer, 0, n, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1000 * layer + loop)
    q = torch.randn(w.batch, w.heads, n, w.D, generator=g, device="cuda").to(torch.bfloat16)
    return q, X[0, loop].contiguous(), X[1, loop].contiguous(), X


def _row_err(got, ref):
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def _run(w, n, lens, label, loop=0):
    B, H, D = w.batch, w.heads, w.D
    q, k, v, _ = _qkv(w, n, loop)
    d = rq.make_desc(B, H, D, w.bits, max(n, 1))
    out = torch.full((B, H, n, D), float("nan"), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = torch.tensor(lens, dtype=torch.int32, device="cuda")
    rq.prefill_attn(d, q, k, v, L, 1.0 / math.sqrt(D), out, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o = out.cpu().double().numpy()
    qn, kn, vn = u16(q), u16(k), u16(v)
    worst = 0.0
    for b in range(B):
        n_b = lens[b]
        assert np.isnan(o[b, :, n_b:]).all(), "rows past the prompt length were written"
        for h in range(H):
            if n_b == 0:
                continue
            ref = O.prefill_attend(qn[b, h, :n_b], kn[b, h, :n_b], vn[b, h, :n_b], 1.0 / math.sqrt(D))
            worst = max(worst, _row_err(o[b, h, :n_b], ref))
    log(f"{label}: max row rel err {worst:.3e}")
    assert worst <= TOL_ATTN, (label, worst)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_prefill_ragged(D):
    """Several query blocks and key tiles, ragged lengths (a block edge, a tile edge,
    one token, empty)."""
    w = synth.WORKLOADS["tiny"].with_(batch=5, heads=2, D=D, nb=32 if D == 96 else 0, outliers=4)
    _run(w, 300, [300, 128, 65, 1, 0], f"prefill D{D}")


def test_prefill_ragged_grouped_order():
    """B8 H2 (B H a multiple of 8): workgroups take the XCD-grouped order, series by
    series; ragged lengths, including empty and one-token sequences."""
    w = synth.WORKLOADS["tiny"].with_(batch=8, heads=2, D=128, outliers=4)
    _run(w, 300, [300, 0, 1, 65, 128, 299, 200, 17], "prefill grouped order")


def test_prefill_long_rows():
    w = synth.WORKLOADS["tiny"].with_(batch=1, heads=2, D=128, outliers=4)
    _run(w, 1500, [1500], "prefill 1500")


def test_prefill_length_flag():
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=1, D=64)
    q, k, v, _ = _qkv(w, 64)
    d = rq.make_desc(2, 1, 64, w.bits, 64)
    out = torch.zeros(2, 1, 64, 64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rq.prefill_attn(d, q, k, v, torch.tensor([64, 99], dtype=torch.int32, device="cuda"), 0.125, out, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == rq.DEVERR_LENGTH
    ref = torch.zeros_like(out)
    rq.prefill_attn(d, q, k, v, torch.tensor([64, 64], dtype=torch.int32, device="cuda"), 0.125, ref)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)              # the long length was clamped to the prompt capacity


def test_prefill_then_store():
    """The whole prefill of the tiny workload: every loop's attention, then the prompt
    quantized into the cache in one bulk append; both against the oracle."""
    w = synth.WORKLOADS["tiny"].with_(batch=2)
    n = 256
    B, H, D, L = w.batch, w.heads, w.D, w.L
    lens = [n, n]
    X = synth.kv(w, 0, 0, n, device="cuda")
    d = rq.make_desc(B, H, D, w.bits, n)
    Ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for r in range(L):
        g = torch.Generator(device="cuda").manual_seed(r)
        q = torch.randn(B, H, n, D, generator=g, device="cuda").to(torch.bfloat16)
        out = torch.empty(B, H, n, D, device="cuda")
        rq.prefill_attn(d, q, X[0, r].contiguous(), X[1, r].contiguous(), Ld, 0.125, out)
        torch.cuda.synchronize()
        o = out.cpu().double().numpy()
        for b in range(B):
            for h in range(H):
                ref = O.prefill_attend(u16(q[b, h]), u16(X[0, r, b, h]), u16(X[1, r, b, h]), 0.125)
                assert _row_err(o[b, h], ref) <= TOL_ATTN
    rk, rv = synth.rotation(w, 0, 0), synth.rotation(w, 0, 1)
    cache = build_gpu_layer(X, rk, rv, w.bits, rq.POLICY_LAST_LOOP, T_max=n, T=n)
    series = oracle_layer(X, rk, rv, w.bits, rq.POLICY_LAST_LOOP, n)
    assert_cache_parity(compare_cache(cache, series, n), "prefill store")


def test_prefill_full_size_sampled_rows():
    """The 16k prompt of the decode benchmark's shape (B8, H16, D128, 16384 tokens), one
    loop: sampled (batch, head) series and rows, through the decode oracle (row i of a
    prefill is a decode step over keys 0..i-1 with token i current)."""
    w = synth.WORKLOADS["ouro_16k"]
    n = w.T
    B, H, D = w.batch, w.heads, w.D
    q, k, v, _ = _qkv(w, n, loop=1)
    d = rq.make_desc(B, H, D, w.bits, n)
    out = torch.empty(B, H, n, D, device="cuda")
    rq.prefill_attn(d, q, k, v, torch.full((B,), n, dtype=torch.int32, device="cuda"), 1.0 / math.sqrt(D), out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 127, 128, 4095, n - 2, n - 1] + rng.integers(0, n, 9).tolist()))
    worst = 0.0
    for (b, h) in [(0, 0), (B - 1, H - 1), (3, 7), (5, 2)]:
        qn, kn, vn = u16(q[b, h]), u16(k[b, h]), u16(v[b, h])
        o = out[b, h].cpu().double().numpy()
        for i in rows:
            ref = O.attend_bf16(kn[:i], vn[:i], qn[i], kn[i], vn[i], 1.0 / math.sqrt(D))
            worst = max(worst, _row_err(o[i][None], ref[None]))
    log(f"prefill 16k: max row rel err {worst:.3e} over {len(rows)} rows x 4 series")
    assert worst <= TOL_ATTN
