"""rq_quantize_append_layers: the appends of several layers in shared launches.

Every layer's buffers must hold exactly the bytes that the one-layer call
writes: contiguous and paged caches, the three reference policies, groups of
16 channels, loop groups, 8 and 32 loops, layer counts that need several
launches, and the bulk path for more than eight tokens. One stack stored this
way is also compared with the oracle.
"""
import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import assert_cache_parity, compare_cache, inputs, log, oracle_layer, shuffled_table

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP

# label, D, bits, policy, loop_group, groups, layers, n, block size (0: contiguous)
CASES = [
    ("last-20-layers", 128, [4, 2, 2, 2], LAST, 0, 32, 20, 1, 0),      # 16 layers per launch: 2 launches
    ("prev-paged", 128, [4, 2, 2, 2], PREV, 0, 32, 3, 1, 16),
    ("first-g16", 96, [4, 2, 2, 2], FIRST, 0, [32, 16, 16, 16], 3, 2, 0),
    ("groups-8-loops", 64, [4, 2, 2, 2, 4, 2, 2, 2], LAST, 4, 32, 10, 1, 0),  # 8 per launch
    ("prev-groups-paged", 128, [4, 2, 4, 2, 4, 2, 4, 2], PREV, 2, 32, 9, 3, 32),
    ("32-loops", 64, [4] + [2] * 31, PREV, 8, 32, 3, 1, 0),              # 2 per launch
    ("bulk-12-tokens", 128, [4, 2, 2, 2], LAST, 0, 32, 2, 12, 0),          # one bulk launch per layer
]


def orthogonal(D: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    q, _ = torch.linalg.qr(torch.randn(D, D, dtype=torch.float64, generator=g))
    return q.float()


def buffers(c: rq.LayerCache):
    out = [c.codes[kv][r] for kv in range(2) for r in range(c.desc.loops)]
    out += [c.meta[kv][r] for kv in range(2) for r in range(c.desc.loops)]
    out += [c.alpha[kv][r] for kv in range(2) for r in range(c.desc.loops) if c.alpha[kv][r] is not None]
    return out


def two_stacks(D, bits, policy, loop_group, groups, nl, B, H, T_max, bs):
    """Two stacks of nl caches with equal rotations and equal (random) contents."""
    table, nb = None, 0
    if bs:
        nb, table = shuffled_table(B, T_max, bs, [T_max] * B, seed=7)
    d = rq.make_desc(B, H, D, bits, T_max, policy, group=groups, loop_group=loop_group, block_size=bs,
                     num_blocks=nb)
    g = torch.Generator(device="cuda").manual_seed(11)
    a, b = [], []
    for l in range(nl):
        rk = torch.stack([orthogonal(D, 1000 * l + 2 * h) for h in range(H)])
        rv = torch.stack([orthogonal(D, 1000 * l + 2 * h + 1) for h in range(H)])
        ca = rq.LayerCache.allocate(d, rk, rv, block_table=table)
        cb = rq.LayerCache.allocate(d, rk, rv, block_table=table)
        for x, y in zip(buffers(ca), buffers(cb)):
            x.view(torch.uint8).copy_(torch.randint(0, 256, x.view(torch.uint8).shape, generator=g,
                                                    device="cuda", dtype=torch.uint8))
            y.copy_(x)
        a.append(ca)
        b.append(cb)
    return d, a, b


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layers_equal_one_layer_calls(case):
    label, D, bits, policy, lg, groups, nl, n, bs = case
    B, H, T_max = 3, 2, 64
    L = len(bits)
    d, one, many = two_stacks(D, bits, policy, lg, groups, nl, B, H, T_max, bs)
    g = torch.Generator(device="cuda").manual_seed(5)
    kv = (3.0 * torch.randn(nl, 2, L, B, H, n, D, generator=g, device="cuda")).to(torch.bfloat16)
    pos = torch.tensor([5, 0, T_max - n], dtype=torch.int32, device="cuda")
    for l in range(nl):
        rq.quantize_append(one[l], kv[l].contiguous(), pos, n)
    rq.quantize_append_layers(many, kv, pos, n)
    torch.cuda.synchronize()
    for l in range(nl):
        for x, y in zip(buffers(one[l]), buffers(many[l])):
            assert torch.equal(x, y), f"{label}: layer {l} differs from the one-layer call"
    log(f"append layers {label}: {nl} layers x {n} tokens equal to the one-layer calls")


@pytest.mark.parametrize("bs", [0, 16], ids=["contiguous", "paged"])
def test_layers_multi_unit_workgroups(bs):
    """Enough (sequence, token) units, heads and layers that the shared launch
    gives each workgroup several units in turn (the rotation staged once for
    them); positions drop a token past capacity partway through a workgroup's
    units. Every layer equals its one-layer call (which has one unit per
    workgroup) and the drop is flagged by both."""
    B, H, T_max, nl, n = 8, 16, 64, 4, 2
    units = B * n
    assert units * H * 2 * nl >= 4 * 2 * 256        # several units per workgroup on any device of <= 256 CUs
    d, one, many = two_stacks(128, [2, 2, 4, 4], LAST, 0, 32, nl, B, H, T_max, bs)
    g = torch.Generator(device="cuda").manual_seed(11)
    kv = (2.0 * torch.randn(nl, 2, 4, B, H, n, 128, generator=g, device="cuda")).to(torch.bfloat16)
    pos = torch.tensor([0, 7, 30, T_max - 1, 12, T_max - 2, 3, 50], dtype=torch.int32, device="cuda")
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(nl):
        rq.quantize_append(one[l], kv[l].contiguous(), pos, n, dev_err=e1)
    rq.quantize_append_layers(many, kv, pos, n, dev_err=e2)
    torch.cuda.synchronize()
    assert int(e1.item()) == int(e2.item()) == rq.DEVERR_CAPACITY
    for l in range(nl):
        for x, y in zip(buffers(one[l]), buffers(many[l])):
            assert torch.equal(x, y), f"layer {l} differs from the one-layer call"
    log(f"append layers multi-unit ({'paged' if bs else 'contiguous'}): {nl} layers x {units} units equal")


def test_layers_capacity_flag():
    """A token past max_tokens is dropped and flagged, by both calls alike."""
    B, H, T_max, nl = 3, 2, 64, 4
    d, one, many = two_stacks(128, [4, 2, 2, 2], LAST, 0, 32, nl, B, H, T_max, 0)
    kv = torch.randn(nl, 2, 4, B, H, 2, 128, device="cuda").to(torch.bfloat16)
    pos = torch.tensor([3, T_max - 1, T_max], dtype=torch.int32, device="cuda")
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(nl):
        rq.quantize_append(one[l], kv[l].contiguous(), pos, 2, dev_err=e1)
    rq.quantize_append_layers(many, kv, pos, 2, dev_err=e2)
    torch.cuda.synchronize()
    assert int(e1.item()) == int(e2.item()) == rq.DEVERR_CAPACITY
    for l in range(nl):
        for x, y in zip(buffers(one[l]), buffers(many[l])):
            assert torch.equal(x, y)


def test_layers_against_oracle():
    """Two layers: tokens [0, T) stored per layer, token T through the shared call;
    each layer's whole cache against the oracle's."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=128, outliers=4)
    B, H, D, L, T, T_max = w.batch, w.heads, w.D, w.L, 100, 128
    stack, data = [], []
    for l in range(2):
        X, rk, rv = inputs(w, T + 1, layer=l, batch=B)
        d = rq.make_desc(B, H, D, list(w.bits), T_max, LAST)
        c = rq.LayerCache.allocate(d, rk, rv)
        rq.quantize_append(c, X[..., :T, :].contiguous(), torch.zeros(B, dtype=torch.int32, device="cuda"), T)
        stack.append(c)
        data.append((X, rk, rv))
    kv = torch.stack([X[..., T:T + 1, :] for X, _, _ in data]).contiguous()
    rq.quantize_append_layers(stack, kv, torch.full((B,), T, dtype=torch.int32, device="cuda"), 1)
    torch.cuda.synchronize()
    for l, (X, rk, rv) in enumerate(data):
        series = oracle_layer(X, rk, rv, list(w.bits), LAST, T + 1)
        assert_cache_parity(compare_cache(stack[l], series, T + 1), f"append layers, layer {l}")
