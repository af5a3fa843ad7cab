"""GPU parity of Previous-loop chains longer than four stored components (paper
"KV Cache Quantization for Looped Transformers with 2-Bit Residuals", App. D
"Logical reference count": decoding loop j of a chain reads j components;
§3.2 "Reference KV"): the cache and every loop's attention against the oracle."""
import pytest
import torch

import decode_attention_quantize_amd as rq
import synth
from rq_parity import (assert_cache_parity, build_gpu_layer, compare_cache, decode_and_compare, inputs, log,
                       oracle_layer)

pytestmark = pytest.mark.gpu

PREV = rq.POLICY_PREV_LOOP


@pytest.mark.parametrize("D,bits", [
    (96, (4, 4, 2, 2, 2, 2, 2, 2)),      # the Huginn-shaped chained comparator's plan
    (128, (4, 2, 2, 2, 2, 2, 2)),
    (64, (2, 2, 2, 2, 2, 2, 2, 2)),
    (128, (4, 4, 2, 2, 2)),
])
def test_long_chain_every_loop(D, bits):
    L = len(bits)
    w = synth.WORKLOADS["huginn_4k"].with_(batch=2, heads=3, D=D, L=L, nb=32 if D == 96 else D, bits=bits,
                                           chained_bits=bits)
    T = 333
    X, rk, rv = inputs(w, T + 1, batch=2)
    label = f"chain D{D} bits={bits}"
    cache = build_gpu_layer(X, rk, rv, bits, PREV, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, bits, PREV, T)
    assert_cache_parity(compare_cache(cache, series, T), label)
    decode_and_compare(w, X, rk, rv, cache, series, [T, 100], range(L), label)


def test_long_chain_precise_query():
    """The 21-bit query instances of a long chain (loop 8 of 8 reads eight components)."""
    bits = (4, 4, 2, 2, 2, 2, 2, 2)
    w = synth.WORKLOADS["huginn_4k"].with_(batch=1, heads=2)
    T = 200
    X, rk, rv = inputs(w, T + 1, batch=1)
    cache = build_gpu_layer(X, rk, rv, bits, PREV, T_max=T + 1, T=T)
    series = oracle_layer(X, rk, rv, bits, PREV, T)
    decode_and_compare(w, X, rk, rv, cache, series, [T], [7, 4], "chain precise", flags=rq.FLAG_PRECISE_QUERY)
