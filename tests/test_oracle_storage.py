"""Pin the storage / traffic calculator to the numbers the pages print
(tests/golden/paper_storage.txt, each line cited there)."""
import os

import pytest

from oracle import storage as S

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    vals = {}
    with open(os.path.join(HERE, "golden", "paper_storage.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


G = _golden()
# The pages' accounting implies 16 metadata bits per group and BF16 (16-bit) LS coefficients.
M = 16


def _round(x, digits):
    return round(x + 1e-12, digits)


@pytest.mark.parametrize("key,bits,group,residual", [
    ("beff_direct_int2_g32", [2, 2, 2, 2], 32, False),
    ("beff_direct_int2_g16", [2, 2, 2, 2], 16, False),
    ("beff_direct_mixed_g32", [2, 2, 2, 4], 32, False),
    ("beff_direct_mixed_g16", [2, 2, 2, 4], [16, 16, 16, 32], False),
    ("beff_residual_int2_g32", [2, 2, 2, 2], 32, True),
    ("beff_residual_int2_g16", [2, 2, 2, 2], 16, True),
    ("beff_residual_mixed_g32", [2, 2, 2, 4], 32, True),
    ("beff_residual_mixed_g16", [2, 2, 2, 4], [16, 16, 16, 32], True),
])
def test_effective_bitwidth(key, bits, group, residual):
    assert _round(S.beff(bits, group, 128, M, 16, residual), 1) == G[key]


def test_alpha_bits():
    assert _round(S.alpha_bits_per_element(4, 128), 3) == G["alpha_extra_bits"]


def test_storage_ratios():
    b = S.beff([2, 2, 2, 4], 32, 128, M, 16, True)
    assert _round(100 * (1 - b / 16), 1) == G["storage_reduction_pct"]
    assert _round(16 / b, 1) == G["storage_reduction_factor"]
    assert _round(100 * b / 16, 1) == G["storage_fraction_pct"]
    plain = S.beff([2, 2, 2, 2], 32, 128, M, 16, False)
    assert _round(100 * plain / 16, 1) == G["plain_int2_fraction_pct"]
    uni = S.beff([2, 2, 2, 2], 32, 128, M, 16, True)
    assert round(100 * (b / uni - 1)) == G["mixed_over_int2_increase_pct"]


def test_logical_access_counts():
    assert S.logical_reads(4, "prev") == G["reads_chain_L4"]
    assert S.logical_reads(4, "last") == G["reads_shared_L4"]
    assert round(S.logical_reads(4, "prev") / S.logical_reads(4, "last"), 2) == G["ratio_L4"]
    assert S.logical_reads(32, "prev") == G["reads_chain_L32"]
    assert S.logical_reads(32, "last") == G["reads_shared_L32"]
    assert round(S.logical_reads(32, "prev") / S.logical_reads(32, "last"), 2) == G["ratio_L32"]
    assert 8 * S.logical_reads(4, "prev") == G["reads_chain_8x4"]
    assert 8 * S.logical_reads(4, "last") == G["reads_shared_8x4"]
    # 32 loops in eight groups of four, counted directly by the grouped model
    assert S.logical_reads(32, "prev", loop_group=4) == G["reads_chain_8x4"]
    assert S.logical_reads(32, "last", loop_group=4) == G["reads_shared_8x4"]
    assert S.logical_reads(32, "first", loop_group=4) == G["reads_shared_8x4"]
    assert S.logical_reads(4, "first") == G["reads_shared_L4"]


def test_decode_bytes_closed_form():
    """Our stored format (fp16 offset + fp16 scale per group of 32, fp16 alpha):
    per head and layer, one token costs INT4 anchor 64+16 = 80 B, INT2 residual
    32+16+2 = 50 B, INT4 residual 64+16+2 = 82 B per tensor. A [2,2,4,4] step reads
    loops 1-2: 2*(80+50), loop 3: 2*(80+82), loop 4: 2*80 -> 1004 B."""
    assert S.decode_bytes_per_token(128, [2, 2, 4, 4]) == 1004
    assert S.decode_bytes_per_token(128, [2, 2, 2, 2]) == 2 * (3 * (48 + 50) + 48)
    # chained [4,4,2,2]: loop1 A; loop2 A+R2(82); loop3 A+R2+R3(50); loop4 A+R2+R3+R4
    assert S.decode_bytes_per_token(128, [4, 4, 2, 2], policy="prev") == 2 * (80 + 162 + 212 + 262)
    assert S.bf16_decode_bytes_per_token(128, 4) == 2048
