"""GPU parity with anchor loop groups and the First-loop policy.

Paper "KV Cache Quantization for Looped Transformers with 2-Bit Residuals":
§5 "Models" (Huginn-3.5B's 32 recurrences as eight independent groups of four,
each group's last loop its anchor), §3.2 "Reference KV" (First-loop: every
other loop refers to the first-loop anchor) and App. D (read counts per
policy). Whole caches and every decoded output are compared with the oracle.
"""
import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, inputs, log, \
    oracle_layer

pytestmark = pytest.mark.gpu

LAST, PREV, FIRST = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP, rq.POLICY_FIRST_LOOP


def _bits(w, policy):
    return w.bits if policy == LAST else w.chained_bits   # INT4 on each group's anchor


def _run(w, policy, T, lens, loops, steps_of_one, chunk, label):
    B = w.batch
    X, rk, rv = inputs(w, T + 1, batch=B)
    bits = _bits(w, policy)
    log(f"{label}: append {T} tokens ({steps_of_one} in chunks of {chunk})")
    cache = build_gpu_layer(X, rk, rv, bits, policy, T_max=T + 1, T=T, steps_of_one=steps_of_one, chunk=chunk,
                            loop_group=w.loop_group)
    series = oracle_layer(X, rk, rv, bits, policy, T, loop_group=w.loop_group)
    assert_cache_parity(compare_cache(cache, series, T), label)
    decode_and_compare(w, X, rk, rv, cache, series, lens, loops, label)


@pytest.mark.parametrize("policy", [LAST, FIRST, PREV])
def test_two_groups_of_four(policy):
    """Eight loops (D96) in two groups of four: a tiled bulk append, then appends of
    one and of three tokens; every loop decoded, one sequence empty of cache."""
    w = synth.WORKLOADS["huginn_4k"].with_(batch=2, heads=3, loop_group=4,
                                            bits=(2, 2, 2, 4) * 2, chained_bits=(4, 2, 2, 2) * 2)
    T = 300
    for chunk in (1, 3):
        _run(w, policy, T, [T, 0], range(8) if chunk == 1 else (), steps_of_one=7, chunk=chunk,
             label=f"8 loops G4 policy={policy} chunk={chunk}")


@pytest.mark.parametrize("policy", [LAST, FIRST])
def test_first_loop_single_group(policy):
    """First-loop and Last-loop over one group of four (D64, [4,2,2,2] and [2,2,2,4])."""
    w = synth.WORKLOADS["tiny"].with_(batch=2, loop_group=0)
    bits = (4, 2, 2, 2) if policy == FIRST else (2, 2, 2, 4)
    w = w.with_(bits=bits, chained_bits=bits)
    _run(w, policy, 257, [257, 100], range(4), steps_of_one=5, chunk=2, label=f"one group policy={policy}")


@pytest.mark.parametrize("policy", [LAST, PREV])
def test_thirty_two_loops(policy):
    """Huginn-shaped 32 loops in eight groups of four (bulk and few-token appends both
    take the per-unit kernel at 32 loops); loops at group edges decoded."""
    w = synth.WORKLOADS["huginn32_4k"].with_(batch=2, heads=2)
    _run(w, policy, 150, [150, 63], (0, 3, 4, 6, 27, 31), steps_of_one=3, chunk=1,
         label=f"32 loops G4 policy={policy}")


def test_loop_groups_of_one():
    """loop_group = 1: every loop is its own anchor (plain group quantization, one
    component per decode)."""
    w = synth.WORKLOADS["tiny"].with_(batch=1, loop_group=1)
    _run(w, LAST, 120, [120], range(4), steps_of_one=2, chunk=1, label="groups of one")
