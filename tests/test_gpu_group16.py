"""GPU parity with INT2 loops in groups of 16 channels (paper §5 "Quantization
setup": g = 16 for INT2, Table 2's g = 16 variants), alone (uniform INT2) and
beside INT4 groups of 32 in one plan, under every reference policy. Whole
caches and every decoded output are compared with the oracle.
"""
import pytest

import decode_attention_quantize_amd as rq
import synth
from rq_parity import assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, inputs, log, \
    oracle_layer

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP


def _run(w, bits, policy, T, lens, steps_of_one, chunk, label, loops=None, groups=None):
    B = w.batch
    groups = groups or [16 if b == 2 else 32 for b in bits]
    X, rk, rv = inputs(w, T + 1, batch=B)
    log(f"{label}: bits {bits} groups {groups}, append {T} tokens ({steps_of_one} in chunks of {chunk})")
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T, steps_of_one=steps_of_one, chunk=chunk,
                            loop_group=w.loop_group, groups=groups)
    series = oracle_layer(X, rk, rv, bits, policy, T, loop_group=w.loop_group, groups=groups)
    assert_cache_parity(compare_cache(cache, series, T), label)
    decode_and_compare(w, X, rk, rv, cache, series, lens, range(len(bits)) if loops is None else loops, label)


@pytest.mark.parametrize("policy,bits", [
    (LAST, (2, 2, 2, 4)),          # INT4 g32 anchor, INT2 g16 residuals
    (LAST, (2, 2, 2, 2)),          # uniform INT2 g16
    (PREV, (4, 2, 2, 2)),          # chained, mixed group sizes in one chain
    (PREV, (4, 4, 2, 2)),          # chained, two INT4 g32 loops before the g16 ones (the 16k chained plan)
    (PREV, (2, 2, 2, 2)),
    (FIRST, (4, 2, 2, 2)),
])
def test_tiny_group16(policy, bits):
    w = synth.WORKLOADS["tiny"].with_(batch=2)
    _run(w, bits, policy, 300, [300, 77], steps_of_one=6, chunk=1, label=f"tiny g16 policy={policy}")


@pytest.mark.parametrize("policy,bits,groups", [
    (LAST, (4, 4, 4, 2), (32, 32, 32, 16)),     # INT2 g16 anchor, INT4 residuals (plan 0x4A)
    (FIRST, (2, 2, 2, 2), (16, 32, 32, 32)),    # g16 anchor, g32 residuals (0x2A)
    (LAST, (2, 2, 2, 2), (16, 16, 16, 32)),     # g32 anchor, g16 residuals (0xA2)
    (PREV, (4, 4, 4, 2), (32, 32, 32, 32)),     # chain with three INT4 loops first (0x2444)
    (PREV, (4, 4, 4, 2), (32, 32, 32, 16)),     # the same, last loop in groups of 16 (0xA444)
])
def test_mixed_group_plans(policy, bits, groups):
    """Plans that mix group sizes between the anchor and the residuals, and chains
    with three INT4 loops before an INT2 one: every loop decoded against the oracle."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, heads=2, D=128, nb=128, outliers=4)
    _run(w, bits, policy, 260, [260, 45], steps_of_one=3, chunk=1,
         label=f"mixed groups policy={policy} bits={bits} groups={groups}", groups=list(groups))


@pytest.mark.parametrize("D", [96, 128])
def test_group16_ragged(D):
    """D96 (three blocks) and D128, ragged lengths including 0 and a tile edge, chunked appends."""
    w = synth.WORKLOADS["tiny"].with_(batch=4, heads=3, D=D, nb=32 if D == 96 else 0, outliers=4)
    T = 500
    _run(w, (2, 2, 4, 4), LAST, T, [0, 1, 2 * 64 // (D // 32) + 1, T], steps_of_one=11, chunk=3,
         label=f"D{D} g16 ragged")


def test_group16_with_loop_groups():
    """Groups of 16 channels inside anchor loop groups (8 loops in two groups of four)."""
    w = synth.WORKLOADS["huginn_4k"].with_(batch=2, heads=2, loop_group=4)
    _run(w, (2, 2, 2, 4) * 2, LAST, 200, [200, 31], steps_of_one=2, chunk=1, label="g16 in loop groups")


def test_group16_at_32_loops():
    """32 loops (the per-unit append kernel for every append) with INT2 groups of 16."""
    w = synth.WORKLOADS["huginn32_4k"].with_(batch=1, heads=2)
    _run(w, w.chained_bits, PREV, 90, [90], steps_of_one=1, chunk=1, label="g16 32 loops", loops=(0, 3, 13, 31))
