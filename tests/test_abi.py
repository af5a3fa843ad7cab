"""The C-ABI library loads, exports every symbol include/rq.h declares, and its
host-side validation rejects bad arguments before enqueuing anything (CPU only:
every call below fails validation, so no GPU work is ever issued)."""
import ctypes
import os
import re

import pytest
import torch

import decode_attention_quantize_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first


def _declared():
    src = open(os.path.join(ROOT, "include", "rq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"rq_quantize_append", "rq_decode_attn", "rq_decode_attn_bf16"} <= set(names)
    lib = ctypes.CDLL(rq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert "gfx950" in rq.version()
    for code in range(12):
        assert rq.status_str(code) and rq.status_str(code) != "unknown status"


def _desc(**kw):
    a = dict(batch=2, heads=3, head_dim=128, bits=[2, 2, 4, 4], max_tokens=100)
    a.update(kw)
    return rq.make_desc(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=80), 2), (dict(batch=0), 2), (dict(max_tokens=0), 2), (dict(bits=[2, 3, 4]), 3),
    (dict(bits=[2] * 33), None), (dict(policy=5), 8), (dict(policy=3), 8), (dict(policy=2), 0),
    (dict(bits=[2] * 32), 0), (dict(loop_group=2), 0), (dict(loop_group=4), 0), (dict(loop_group=1), 0),
    (dict(loop_group=3), 2), (dict(loop_group=5), 2), (dict(loop_group=-1), 2),
    (dict(bits=[2] * 32, loop_group=4), 0), (dict(bits=[2] * 32, loop_group=12), 2),
    (dict(flags=1), 0), (dict(flags=2), 0), (dict(flags=3), 0), (dict(flags=4), 2), (dict(flags=-1), 2),
])
def test_check_desc(kw, code):
    if code is None:
        with pytest.raises(IndexError):
            _desc(**kw)
        return
    assert rq.check_desc(_desc(**kw)) == code


def test_desc_layout_matches_header(tmp_path):
    """The ctypes mirrors of rq_desc and rq_layer_cache have the sizes and field offsets
    a C compiler gives the structs of include/rq.h."""
    import subprocess
    fields = {"rq_desc": [f for f, _ in rq.Desc._fields_], "rq_layer_cache": [f for f, _ in rq.LayerCacheC._fields_]}
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "rq.h"', "int main(void) {"]
    for st, fs in fields.items():
        prog.append(f'  printf("{st} size %zu\\n", sizeof({st}));')
        for f in fs:
            prog.append(f'  printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    prog += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        st, f, v = line.split()
        got[(st, f)] = int(v)
    assert got[("rq_desc", "size")] == ctypes.sizeof(rq.Desc)
    assert got[("rq_layer_cache", "size")] == ctypes.sizeof(rq.LayerCacheC)
    for f in fields["rq_desc"]:
        assert got[("rq_desc", f)] == getattr(rq.Desc, f).offset, f
    for f in fields["rq_layer_cache"]:
        assert got[("rq_layer_cache", f)] == getattr(rq.LayerCacheC, f).offset, f
    assert rq.MAX_LOOPS == 32


@pytest.mark.parametrize("bs,nb,code", [
    (16, 10, 0), (64, 1, 0), (4096, 3, 0), (0, 0, 0), (8, 10, 2), (48, 10, 2), (8192, 1, 2), (16, 0, 2),
    (-16, 4, 2),
])
def test_paged_desc_validation(bs, nb, code):
    assert rq.check_desc(_desc(max_tokens=8192, block_size=bs, num_blocks=nb)) == code


def test_paged_block_size_divides_max_tokens():
    assert rq.check_desc(_desc(max_tokens=1056, block_size=32, num_blocks=4)) == 0      # 33 blocks
    assert rq.check_desc(_desc(max_tokens=1048, block_size=32, num_blocks=4)) == 2


def test_paged_pool_size_limit():
    """Every pool buffer must stay addressable by 32-bit offsets (INT4 codes are the largest)."""
    ok = _desc(block_size=16, num_blocks=(0xFFFF0000 // (64 * 3 * 16)), max_tokens=1024)
    assert rq.check_desc(ok) == 0
    big = _desc(block_size=16, num_blocks=(0xFFFF0000 // (64 * 3 * 16)) + 1, max_tokens=1024)
    assert rq.check_desc(big) == 2


def test_paged_buffer_bytes():
    d = _desc(block_size=64, num_blocks=7, max_tokens=1024)     # bits [2, 2, 4, 4], H3, D128
    rows = 7 * 3 * 64
    assert rq.buffer_bytes(d, 0, 0) == rows * 32
    assert rq.buffer_bytes(d, 0, 3) == rows * 64
    assert rq.buffer_bytes(d, 1, 1) == rows * 4 * 4
    assert rq.buffer_bytes(d, 2, 0) == rows * 2


def test_paged_calls_need_the_table():
    L, by = rq.lib, ctypes.byref
    d = _desc(block_size=16, num_blocks=40, max_tokens=1024)
    c = _cache(d)
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 1         # no table
    ws = rq.workspace_bytes(d)
    assert L.rq_decode_attn(by(d), by(c), 0, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, ws,
                            None, 0) == 1
    c.block_table = 0x100002
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 10
    assert L.rq_decode_attn(by(d), by(c), 0, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, ws,
                            None, 0) == 10


@pytest.mark.parametrize("policy,G,L,expect", [
    (0, 0, 4, [3, 3, 3, 3]), (2, 0, 4, [0, 0, 0, 0]), (1, 0, 4, [0, 0, 0, 0]),
    (0, 4, 8, [3, 3, 3, 3, 7, 7, 7, 7]), (2, 4, 8, [0, 0, 0, 0, 4, 4, 4, 4]), (1, 2, 4, [0, 0, 2, 2]),
    (0, 1, 3, [0, 1, 2]),
])
def test_anchor_of(policy, G, L, expect):
    d = _desc(bits=[2] * L, policy=policy, loop_group=G)
    assert [rq.anchor_of(d, r) for r in range(L)] == expect


def test_group_sizes():
    """Groups of 32 everywhere, or 16 for 2-bit loops (INT4 stays at 32)."""
    d = _desc()                                   # bits [2, 2, 4, 4]
    d.group[1] = 16
    assert rq.check_desc(d) == 0
    d.group[2] = 16
    assert rq.check_desc(d) == 3
    d.group[2] = 32
    d.group[0] = 64
    assert rq.check_desc(d) == 3
    d.group[0] = 8
    assert rq.check_desc(d) == 3
    assert rq.check_desc(_desc(group=[16, 16, 32, 32])) == 0
    assert rq.buffer_bytes(_desc(group=[16, 16, 32, 32]), 1, 0) == 2 * 3 * 100 * 8 * 4
    with pytest.raises(ValueError):
        _desc(group=[16, 32])


def test_group16_meta_alignment():
    """Metadata of a loop in groups of 16 is read 8 bytes at a time: 8-byte alignment."""
    L, by = rq.lib, ctypes.byref
    d = _desc(group=[16, 16, 32, 32])
    c = _cache(d)
    c.meta[1][0] = 0x100004                       # 4-byte aligned only
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 10
    ws = rq.workspace_bytes(d)
    assert L.rq_decode_attn(by(d), by(c), 0, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, ws,
                            None, 0) == 10
    c.meta[1][0] = 0x100000
    c.meta[1][2] = 0x100004                       # groups of 32: 4 bytes suffice, the next check fails
    c.codes[1][3] = 0x100004
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 10


def test_decode_support_rule():
    """rq_check_decode (host only) against the documented rule, over every 4-loop plan of
    widths and group sizes, all three policies, contiguous and paged: one or two
    components always; chains whose INT4 loops precede their INT2 loops, the INT2 loops
    in one group size. Chains of 5-8: contiguous, at most two INT4 loops first, groups of 32."""
    import itertools
    kinds = [(2, 32), (2, 16), (4, 32)]
    for pol in (rq.POLICY_LAST_LOOP, rq.POLICY_FIRST_LOOP, rq.POLICY_PREV_LOOP):
        for bs in (0, 16):
            for combo in itertools.product(kinds, repeat=4):
                kw = dict(block_size=bs, num_blocks=64, max_tokens=128) if bs else {}
                d = _desc(bits=[k[0] for k in combo], group=[k[1] for k in combo], policy=pol, **kw)
                assert rq.check_desc(d) == 0
                for r in range(4):
                    if pol == rq.POLICY_PREV_LOOP:
                        ks = combo[:r + 1]
                        wide = [k[0] == 4 for k in ks]
                        ok = len(ks) <= 2 or (wide == sorted(wide, reverse=True)
                                              and len({k[1] for k in ks if k[0] == 2}) <= 1)
                    else:
                        ok = True
                    assert rq.check_decode(d, r) == (0 if ok else 6), (pol, bs, combo, r)
    for bits, ok in (([4, 4] + [2] * 6, True), ([4] + [2] * 7, True), ([2] * 8, True), ([4, 4, 4] + [2] * 5, False),
                     ([2, 4] + [2] * 6, False)):
        d = _desc(bits=bits, policy=rq.POLICY_PREV_LOOP)
        assert rq.check_decode(d, 7) == (0 if ok else 6), bits
        d16 = _desc(bits=bits, group=[16 if b == 2 else 32 for b in bits], policy=rq.POLICY_PREV_LOOP)
        assert rq.check_decode(d16, 7) == 6
        dp = _desc(bits=bits, policy=rq.POLICY_PREV_LOOP, block_size=16, num_blocks=64, max_tokens=128)
        head = [b == 4 for b in bits[:4]]
        assert rq.check_decode(dp, 4) == 6 and rq.check_decode(dp, 3) == (0 if head == sorted(head, reverse=True) else 6)
    d = _desc()
    assert rq.check_decode(d, 4) == 9 and rq.check_decode(d, -1) == 9
    assert rq.check_decode(_desc(head_dim=80), 0) == 2


def test_buffer_and_workspace_sizes():
    d = _desc()
    toks = 2 * 3 * 100
    assert rq.buffer_bytes(d, 0, 0) == toks * 128 * 2 // 8
    assert rq.buffer_bytes(d, 0, 3) == toks * 128 * 4 // 8
    assert rq.buffer_bytes(d, 1, 2) == toks * 4 * 4
    assert rq.buffer_bytes(d, 2, 1) == toks * 2
    assert rq.buffer_bytes(d, 0, 4) == 0 and rq.buffer_bytes(d, 7, 0) == 0
    assert rq.workspace_bytes(d) > 0
    bad = _desc(head_dim=80)
    assert rq.workspace_bytes(bad) == 0


def _cache(d, null_alpha=False):
    c = rq.LayerCacheC()
    for kv in range(2):
        for r in range(d.loops):
            c.codes[kv][r] = 0x100000
            c.meta[kv][r] = 0x100000
            c.alpha[kv][r] = None if null_alpha else 0x100000
        c.rot[kv] = 0x100000
    return c


def test_append_validation():
    L = rq.lib
    d = _desc()
    c = _cache(d)
    by = ctypes.byref
    assert L.rq_quantize_append(None, by(c), FAKE, FAKE, 1, None, 0) == 1
    assert L.rq_quantize_append(by(d), None, FAKE, FAKE, 1, None, 0) == 1
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, -1, None, 0) == 2
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 101, None, 0) == 4
    assert L.rq_quantize_append(by(d), by(c), None, FAKE, 1, None, 0) == 1
    assert L.rq_quantize_append(by(d), by(c), FAKE, None, 1, None, 0) == 1
    assert L.rq_quantize_append(by(d), by(c), None, None, 0, None, 0) == 0      # n == 0: no-op
    cn = _cache(d, null_alpha=True)                                            # residual loops need alpha
    assert L.rq_quantize_append(by(d), by(cn), FAKE, FAKE, 1, None, 0) == 1
    ca = _cache(d)
    ca.meta[0][1] = 0x100002                                                   # meta needs 4 bytes
    assert L.rq_quantize_append(by(d), by(ca), FAKE, FAKE, 1, None, 0) == 10
    assert L.rq_quantize_append(by(d), by(c), ctypes.c_void_p(0x100001), FAKE, 1, None, 0) == 10


def test_append_layers_validation():
    """Every layer is checked before the first launch (no call here reaches one)."""
    L, by = rq.lib, ctypes.byref
    d = _desc()
    arr = (rq.LayerCacheC * 3)(_cache(d), _cache(d), _cache(d))
    assert L.rq_quantize_append_layers(by(d), None, 3, FAKE, FAKE, 1, None, 0) == 1
    assert L.rq_quantize_append_layers(by(d), arr, -1, FAKE, FAKE, 1, None, 0) == 2
    assert L.rq_quantize_append_layers(by(d), arr, 0, FAKE, FAKE, 1, None, 0) == 0     # no layers: no-op
    assert L.rq_quantize_append_layers(by(d), arr, 3, None, None, 0, None, 0) == 0     # n == 0: no-op
    assert L.rq_quantize_append_layers(by(d), arr, 3, FAKE, FAKE, 101, None, 0) == 4
    assert L.rq_quantize_append_layers(by(d), arr, 3, None, FAKE, 1, None, 0) == 1
    arr[2].meta[1][1] = 0x100002                                                     # last layer misaligned
    assert L.rq_quantize_append_layers(by(d), arr, 3, FAKE, FAKE, 1, None, 0) == 10
    arr[2].meta[1][1] = 0x100000
    arr[1].alpha[0][2] = None                                                        # a residual without alpha
    assert L.rq_quantize_append_layers(by(d), arr, 3, FAKE, FAKE, 1, None, 0) == 1


def test_append_layers_binding_checks():
    """The binding refuses caches with different descriptors and a kv of the wrong shape."""
    d1, d2 = _desc(), _desc(max_tokens=200)
    a = rq.LayerCache(d1, [], [], [], [])
    b = rq.LayerCache(d2, [], [], [], [])
    kv = torch.zeros(2, 2, d1.loops, d1.batch, d1.heads, 1, d1.head_dim, dtype=torch.bfloat16)
    pos = torch.zeros(d1.batch, dtype=torch.int32)
    with pytest.raises(ValueError, match="descriptor differs"):
        rq.quantize_append_layers([a, b], kv, pos, 1)
    with pytest.raises(ValueError, match="kv"):
        rq.quantize_append_layers([a, a, a], kv, pos, 1)


@pytest.mark.parametrize("policy", [0, 1, 2])
def test_append_validation_groups(policy):
    """With loop groups only each group's anchor may go without an alpha buffer. A
    misaligned buffer in the last loop of the value tensor shows that the checks got
    past every alpha pointer (no call here reaches a launch)."""
    L, by = rq.lib, ctypes.byref
    d = _desc(bits=[2] * 8, policy=policy, loop_group=4)
    anchors = {rq.anchor_of(d, r) for r in range(8)}
    assert len(anchors) == 2
    c = _cache(d)
    for kv in range(2):
        for r in anchors:
            c.alpha[kv][r] = None
    c.codes[1][7] = 0x100004
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 10
    r_res = next(r for r in range(8) if r not in anchors)
    c.alpha[0][r_res] = None
    assert L.rq_quantize_append(by(d), by(c), FAKE, FAKE, 1, None, 0) == 1


def test_decode_validation():
    L = rq.lib
    d = _desc()
    c = _cache(d)
    by = ctypes.byref
    ws = rq.workspace_bytes(d)
    args = lambda loop=0, q=FAKE, ws_ptr=FAKE, ws_n=ws, scale=0.1: (
        by(d), by(c), loop, q, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE, ws_ptr, ws_n, None, 0)
    assert L.rq_decode_attn(*args(loop=4)) == 9
    assert L.rq_decode_attn(*args(loop=-1)) == 9
    assert L.rq_decode_attn(*args(q=None)) == 1
    assert L.rq_decode_attn(*args(ws_ptr=None)) == 5
    assert L.rq_decode_attn(*args(ws_n=ws - 1)) == 5
    assert L.rq_decode_attn(*args(ws_ptr=ctypes.c_void_p(0x100010))) == 5    # not 256-byte aligned
    assert L.rq_decode_attn(*args(scale=float("nan"))) == 2
    assert L.rq_decode_attn(*args(q=ctypes.c_void_p(0x100008))) == 10        # q needs 16-byte alignment
    cm = _cache(d)
    cm.codes[1][3] = 0x100004                                                  # codes need 16 bytes
    assert L.rq_decode_attn(by(d), by(cm), 0, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, ws,
                            None, 0) == 10
    # chained policy with more components than the fused kernel takes (9), a long chain of
    # an order without an instance (INT2 anchor, then INT4), and a long chain in a paged cache
    for bits, loop, kw in (([2] * 9, 8, {}), ([2, 4, 2, 4, 2, 4], 5, {}),
                           ([4, 2, 2, 2, 2], 4, dict(block_size=16, num_blocks=40, max_tokens=1024))):
        dl = _desc(bits=bits, policy=1, **kw)
        cl = _cache(dl)
        if kw:
            cl.block_table = 0x100000
        assert L.rq_decode_attn(by(dl), by(cl), loop, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                rq.workspace_bytes(dl), None, 0) == 6, (bits, kw)
    # chains restart in every loop group: loop 13 of 32 in groups of 16 reads loops 0..13
    d16 = _desc(bits=[2] * 32, policy=1, loop_group=16)
    c16 = _cache(d16)
    assert L.rq_decode_attn(by(d16), by(c16), 13, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                            rq.workspace_bytes(d16), None, 0) == 6
    # a shared-anchor read of loop 13 in groups of 8 takes the group's anchor, then loop 13:
    # a misaligned anchor buffer is reported before loop 13's missing meta, and loop 0 (NULL
    # codes) is never read; every call ends in an error before any launch
    for policy, anchor in ((0, 15), (2, 8)):
        dg = _desc(bits=[2] * 16, policy=policy, loop_group=8)
        cg = _cache(dg)
        cg.codes[0][0] = None
        cg.meta[1][13] = None
        cg.codes[1][anchor] = 0x100004
        assert L.rq_decode_attn(by(dg), by(cg), 13, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                rq.workspace_bytes(dg), None, 0) == 10
        cg.codes[1][anchor] = 0x100000
        assert L.rq_decode_attn(by(dg), by(cg), 13, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                rq.workspace_bytes(dg), None, 0) == 1


def test_prefill_validation():
    L, by = rq.lib, ctypes.byref
    d = _desc()
    f = ctypes.c_float(0.1)
    ws = rq.prefill_workspace_bytes(d, 8)
    assert ws == 2 * 3 * 128 * 64 * 2                     # B H D x 8 keys padded to one 64-key tile, fp16
    assert rq.prefill_workspace_bytes(d, 65) == 2 * 3 * 128 * 128 * 2
    args = lambda n=8, q=FAKE, k=FAKE, lens=FAKE, out=FAKE, scale=f, ws_ptr=FAKE, ws_n=ws: (
        by(d), q, k, FAKE, lens, n, scale, out, ws_ptr, ws_n, None, 0)
    assert L.rq_prefill_attn(None, FAKE, FAKE, FAKE, FAKE, 8, f, FAKE, FAKE, ws, None, 0) == 1
    assert L.rq_prefill_attn(*args(n=-1)) == 2
    assert L.rq_prefill_attn(by(d), None, None, None, None, 0, f, None, None, 0, None, 0) == 0   # n == 0: no-op
    assert L.rq_prefill_attn(*args(q=None)) == 1
    assert L.rq_prefill_attn(*args(lens=None)) == 1
    assert L.rq_prefill_attn(*args(out=None)) == 1
    assert L.rq_prefill_attn(*args(k=ctypes.c_void_p(0x100008))) == 10
    assert L.rq_prefill_attn(*args(out=ctypes.c_void_p(0x100004))) == 10
    assert L.rq_prefill_attn(*args(scale=ctypes.c_float(float("inf")))) == 2
    assert L.rq_prefill_attn(*args(scale=ctypes.c_float(0.0))) == 2
    assert L.rq_prefill_attn(*args(scale=ctypes.c_float(-0.1))) == 2
    assert L.rq_prefill_attn(*args(ws_ptr=None)) == 5
    assert L.rq_prefill_attn(*args(ws_n=ws - 1)) == 5
    assert L.rq_prefill_attn(*args(ws_ptr=ctypes.c_void_p(0x100010))) == 5
    assert L.rq_prefill_attn(by(_desc(head_dim=80)), FAKE, FAKE, FAKE, FAKE, 8, f, FAKE, FAKE, ws, None, 0) == 2


@pytest.mark.parametrize("B,H,D,T,expect", [
    (2, 3, 128, 100, 1),          # shorter than 8 tiles: one slot
    (1, 16, 128, 4160, 16),       # 4160 // (32 * 8): capped below the 48 slots three per CU would give
    (8, 16, 128, 16448, 6),       # ceil(3 * 256 / 128): the 16k benchmark shape
    (4, 55, 96, 4160, 2),         # ceil(3 * 256 / 220) = 4 overshoots 768: floor(2 * 256 / 220)
    (2, 3, 128, 65600, 128),      # ceil(768 / 6) = 128 fits exactly
    (2, 7, 128, 65600, 36),       # ceil(768 / 14) = 55 overshoots: floor(512 / 14)
    (128, 16, 128, 8256, 1),      # more series than workgroup slots
])
def test_split_plan_rule(B, H, D, T, expect):
    """Split plan: about three workgroups per compute unit (256 CUs here, the
    count the library assumes without a device), or two where rounding up would
    overshoot three, but every slot at least 8 tiles of the capacity."""
    d = rq.make_desc(B, H, D, [2, 2, 4, 4], T)
    unit, nsplit = rq.split_plan(d)
    assert unit == 2 * 64 // (D // 32)
    if rq_cus() == 256:
        assert nsplit == expect
    assert 1 <= nsplit <= max(1, T // (unit * 8))


def rq_cus():
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.get_device_properties(0).multi_processor_count
    except Exception:
        pass
    return 256


def test_split_api_validation():
    L = rq.lib
    d = _desc()
    c = _cache(d)
    by = ctypes.byref
    ws = rq.workspace_bytes(d)
    unit, nsplit = rq.split_plan(d)
    assert unit == 2 * 64 // (d.head_dim // 32) and 1 <= nsplit <= -(-d.max_tokens // unit)
    for n in (0, 1, unit, d.max_tokens):
        sl = rq.slot_len(n, nsplit, unit)
        assert sl % unit == 0 and sl * nsplit >= n and (sl - unit) * nsplit < max(n, 1)
    assert ws == d.batch * d.heads * nsplit * (d.head_dim + 4) * 4
    assert L.rq_split_plan(by(d), None, None) == 1
    f = ctypes.c_float(0.1)
    assert L.rq_decode_attn_partial(by(d), by(c), 4, FAKE, FAKE, f, FAKE, ws, 0) == 9
    assert L.rq_decode_attn_partial(by(d), by(c), 0, None, FAKE, f, FAKE, ws, 0) == 1
    assert L.rq_decode_attn_partial(by(d), by(c), 0, FAKE, FAKE, f, FAKE, ws - 4, 0) == 5
    assert L.rq_decode_attn_partial(by(d), by(c), 0, ctypes.c_void_p(0x100002), FAKE, f, FAKE, ws, 0) == 10
    assert L.rq_decode_combine(by(d), None, FAKE, FAKE, FAKE, FAKE, f, None, FAKE, ws, None, 0) == 1
    assert L.rq_decode_combine(by(d), ctypes.c_void_p(0x100004), FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, ws,
                               None, 0) == 10
    assert L.rq_decode_combine(by(d), None, FAKE, FAKE, FAKE, FAKE, f, FAKE, FAKE, ws - 1, None, 0) == 5
    assert L.rq_decode_combine(by(d), None, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(float("inf")), FAKE, FAKE,
                               ws, None, 0) == 2


def test_bf16_validation():
    L = rq.lib
    d = _desc()
    by = ctypes.byref
    ws = rq.workspace_bytes(d)
    assert L.rq_decode_attn_bf16(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                 ws, None, 0) == 1
    assert L.rq_decode_attn_bf16(by(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                 ws, None, 0) == 1
    assert L.rq_decode_attn_bf16(by(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                                 ws - 1, None, 0) == 5
    f = ctypes.c_float(0.1)
    assert L.rq_decode_attn_bf16_partial(by(d), None, FAKE, FAKE, FAKE, f, FAKE, ws, 0) == 1
    assert L.rq_decode_attn_bf16_partial(by(d), FAKE, FAKE, FAKE, FAKE, f, FAKE, ws - 1, 0) == 5
    assert L.rq_decode_attn_bf16_partial(by(d), FAKE, ctypes.c_void_p(0x100004), FAKE, FAKE, f, FAKE, ws, 0) == 10
    assert L.rq_decode_attn_bf16(by(d), ctypes.c_void_p(0x100008), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 ctypes.c_float(0.1), FAKE, FAKE, ws, None, 0) == 10


def test_binding_checks_tensors_before_the_call():
    """The binding checks every tensor against the descriptor before calling the
    library (raw pointers carry no sizes): a K/V input with too few loops, a wrong
    dtype, a non-contiguous view or a host tensor is refused with an error."""
    import torch
    d = _desc(batch=2, heads=3, head_dim=64, bits=[2, 2, 2, 4], max_tokens=64)
    rk = torch.eye(64).expand(3, 64, 64).contiguous()
    c = rq.LayerCache.allocate(d, rk, rk, device="cpu")
    pos = torch.zeros(2, dtype=torch.int32)
    good = torch.zeros(2, 4, 2, 3, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="kv: expected shape"):
        rq.quantize_append(c, torch.zeros(2, 2, 2, 3, 1, 64, dtype=torch.bfloat16), pos, 1)   # 2 loops, not 4
    with pytest.raises(ValueError, match="kv: expected torch.bfloat16"):
        rq.quantize_append(c, good.float(), pos, 1)
    with pytest.raises(ValueError, match="kv: must be contiguous"):
        rq.quantize_append(c, torch.zeros(2, 4, 2, 3, 1, 128, dtype=torch.bfloat16)[..., ::2], pos, 1)
    with pytest.raises(ValueError, match="pos: expected torch.int32"):
        rq.quantize_append(c, good, pos.long(), 1)
    with pytest.raises(ValueError, match="must be on a GPU device"):
        rq.quantize_append(c, good, pos, 1)
    q = torch.zeros(2, 3, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out: expected shape"):
        rq.decode_attn(c, 0, q, q, q, pos, 0.1, torch.zeros(2, 3, 32), torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="k_cache: expected shape"):
        rq.decode_attn_bf16(d, torch.zeros(2, 3, 63, 64, dtype=torch.bfloat16), None, q, q, q, pos, 0.1,
                            torch.zeros(2, 3, 64), torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="v: expected shape"):
        rq.prefill_attn(d, torch.zeros(2, 3, 8, 64, dtype=torch.bfloat16), torch.zeros(2, 3, 8, 64, dtype=torch.bfloat16),
                        torch.zeros(2, 3, 9, 64, dtype=torch.bfloat16), torch.zeros(2, dtype=torch.int32), 0.1,
                        torch.zeros(2, 3, 8, 64))
    bad = rq.LayerCache.allocate(d, rk, rk, device="cpu")
    bad.codes[0][1] = torch.zeros(5, dtype=torch.uint8)
    with pytest.raises(ValueError, match=r"cache codes\[0\]\[1\]: 5 bytes"):
        bad.validate()
    with pytest.raises(ValueError, match=r"cache codes\[0\]\[0\]: must be on a GPU device"):
        c.validate()


def test_read_calibration_library_validation():
    """The benchmark's read-rate calibration (librq_calib.so) loads, exports its one
    call and rejects arguments outside its limits without a launch."""
    import bench
    lib = bench._calib_lib()
    assert lib is not None, "librq_calib.so is built beside librq.so"
    bufs = (ctypes.c_void_p * 2)(0x100000, 0x200000)

    def call(bpt, n=2, B=8, H=16, T_max=16448, length=16384, nsplit=6, unit=32, sink=FAKE, b=bufs):
        return lib.rqc_read_slots(b, (ctypes.c_int * 2)(*bpt), n, B, H, T_max, length, nsplit, unit, sink, None)
    assert call((0, 16)) == -1
    assert call((1 << 20, 16)) == -1               # a buffer of 2^31 bytes or more per (b, h)
    assert call((32, 16), length=16500) == -1      # longer than T_max
    assert call((32, 16), n=0) == -1
    assert call((32, 16), n=25) == -1              # more buffers than it takes
    assert call((32, 16), nsplit=0) == -1
    assert call((32, 16), unit=0) == -1
    assert call((32, 16), sink=None) == -1
    assert call((32, 16), b=(ctypes.c_void_p * 2)(0x100000, None)) == -1


def test_fp16_rotation_storage_in_the_binding():
    """FLAG_ROT_F16 (rq.h RQ_FLAG_ROT_F16) makes the cache's rotations fp16 tensors; a
    tensor of the other dtype is refused; a per-call decode flag never changes the
    cache's rotation storage."""
    import torch
    d16 = _desc(batch=2, heads=3, head_dim=64, bits=[2, 2, 2, 4], max_tokens=64, flags=rq.FLAG_ROT_F16)
    d32 = _desc(batch=2, heads=3, head_dim=64, bits=[2, 2, 2, 4], max_tokens=64)
    assert rq.check_desc(d16) == 0 and rq.check_decode(d16, 0) == 0
    rk = torch.eye(64).expand(3, 64, 64).contiguous()
    c = rq.LayerCache.allocate(d16, rk, rk, device="cpu")
    assert c.rot[0].dtype == torch.float16 and c.rot[1].dtype == torch.float16
    assert rq.rot_dtype(d16) == torch.float16 and rq.rot_dtype(d32) == torch.float32
    c.rot[1] = rk.clone()
    with pytest.raises(ValueError, match=r"cache rot\[1\]: expected torch.float16"):
        c.validate()
    assert rq._with_flags(d16, rq.FLAG_PRECISE_QUERY).flags == rq.FLAG_PRECISE_QUERY | rq.FLAG_ROT_F16
    assert rq._with_flags(d16, 0).flags == rq.FLAG_ROT_F16
    assert rq._with_flags(d32, rq.FLAG_ROT_F16).flags == 0
    assert rq._with_flags(d16, None) is d16
    q = torch.zeros(2, 3, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rot_v: expected torch.float16"):
        rq.decode_combine(d16, rk, q, q, q, torch.zeros(2, dtype=torch.int32), 0.1, torch.zeros(2, 3, 64),
                          torch.zeros(256, dtype=torch.uint8))
