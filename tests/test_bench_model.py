"""The benchmark's algorithmic byte model against the library's layout (CPU only).

The roofline's `achieved` figure is algorithmic bytes / time, so the bytes per
(b, h, cached token) that bench.py charges each decode call must be exactly
the bytes of the stored components the call reads: here they are checked
against rq_buffer_bytes (the library's own buffer sizes) and against the
16k workload's totals quoted in the design notes.
"""
import pytest

import bench
import decode_attention_quantize_amd as rq

LAST, PREV = rq.POLICY_LAST_LOOP, rq.POLICY_PREV_LOOP


def _lib_bytes_per_token(d, r, with_alpha):
    """Bytes of loop r's stored arrays (K and V) per (b, h, token), from rq_buffer_bytes."""
    rows = d.batch * d.heads * d.max_tokens
    per = sum(rq.buffer_bytes(d, kind, r) for kind in (0, 1)) + (rq.buffer_bytes(d, 2, r) if with_alpha else 0)
    assert per % rows == 0
    return 2 * per // rows


@pytest.mark.parametrize("D,bits,groups,policy,G", [
    (128, [2, 2, 4, 4], [32] * 4, LAST, 0),
    (128, [4, 4, 2, 2], [32, 32, 16, 16], PREV, 0),
    (96, [2, 2, 2, 2, 2, 2, 4, 4], [32] * 8, LAST, 0),
    (96, [2, 2, 2, 4] * 2, [32, 16, 16, 32] * 2, LAST, 4),
    (96, [4, 2, 2, 2] * 2, [32] * 8, PREV, 4),
])
def test_call_bytes_match_the_library_layout(D, bits, groups, policy, G):
    """Last-loop reads the group's anchor plus loop r's residual; Previous-loop reads
    the chain from the group's first loop up to r; alpha only for non-anchors."""
    d = rq.make_desc(2, 3, D, bits, 64, policy, group=groups, loop_group=G)
    name = "last" if policy == LAST else "prev"
    for r in range(len(bits)):
        a = rq.anchor_of(d, r)
        comps = ([a] if r == a else [a, r]) if policy == LAST else list(range(a, r + 1))
        want = sum(_lib_bytes_per_token(d, c, c != a) for c in comps)
        assert bench.call_bytes(D, bits, name, r, G, groups) == want, (r, want)


def test_default_workload_totals():
    """16k workload, plan [2,2,4,4], Last-loop: 260, 260, 324 and 160 bytes per (b, h,
    token) for loops 1-4 (INT4 anchor 64 + 16 bytes per tensor; INT2 residual 32 + 16
    + 2; INT4 residual 64 + 16 + 2), 385,536 bytes per cached token and sequence over
    24 layers and 16 heads, 545,259,520 bytes for one loop-1 call at 16,384 tokens,
    B8, H16; the chained comparator's [4,4,2,2] chains read 160, 324, 424 and 524."""
    bits = [2, 2, 4, 4]
    per = [bench.call_bytes(128, bits, "last", r) for r in range(4)]
    assert per == [260, 260, 324, 160]
    assert sum(per) * 16 * 24 == 385536
    assert per[0] * 8 * 16 * 16384 == 545259520
    assert [bench.call_bytes(128, [4, 4, 2, 2], "prev", r) for r in range(4)] == [160, 324, 424, 524]
    assert bench.dom_kernel_name(128, bits, 0) == "decode_fused<128, 2, 36u, 2, 2, 1>"
    assert bench.dom_kernel_name(128, bits, 0, rot16=False) == "decode_fused<128, 2, 36u, 2, 2, 0>"
