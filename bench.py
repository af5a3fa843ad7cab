#!/usr/bin/env python3
"""Decode-attention benchmark of the ResidualQuant path on one MI355X.

Workload (default "ouro_16k"): Ouro-1.4B-shaped looped decoder, 24 layers,
batch 8, 16 MHA heads, head_dim 128, 4 loops, 16384 cached tokens, INT2/4
plan [2,2,4,4] (loops 1-2 INT2 residuals, loop 3 INT4 residual, INT4 anchor),
group 32, synthetic seeded inputs (synth/). One step = one decoded token per
sequence: for each loop r and layer l, rq_decode_attn over the compressed
cache with the current token's bf16 K/V; after the final loop, one
rq_quantize_append_layers call stores the current token (all loops) of every
layer at position past_len; then past_len += 1 on the device. Each step is one
captured hipGraph.

Reported next to it, in the same process and on the same logical inputs:
  * the BF16 decode baseline (rq_decode_attn_bf16 over the uncompressed cache);
  * the chained Previous-loop reference policy ([4,4,2,2], anchor on loop 1);
  * per-call HIP-event timing of the dominant call for the roofline (and of the
    same launch with the 21-bit rotated query);
  * the prefill attention of one loop and the bulk store of the prompt;
  * "configs": compact records of the other workload shapes (uniform INT2 at
    4k, B1; the Huginn-shaped recurrence, B4, 4k; the 8k capacity shape with
    RQ at batch 128 against BF16 at batch 32, its largest that fits), each with
    16 decode steps;
  * the CPU oracle timed on a bounded sample (cpu_baseline).

Other workloads of synth.WORKLOADS run with --workload, e.g. "huginn32_4k"
(32 recurrences in eight anchor groups of four, D96, 55 heads); per-call
timings then cover the loops of one group, and the counter-based traffic
figure (taken for the default workload only) is null.

Prints one JSON line (rank 0). --gpus N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s + achieved HBM GB/s (% of peak) at 16k ctx, 4 loops"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0            # dense bf16 matrix-core peak of the MI355X
FP64_PEAK_TFLOPS = 78.6             # fp64 matrix-core peak of the MI355X


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- traffic model
def comp_bytes(D, bits, with_alpha, group=32):
    return D * bits // 8 + (D // group) * 4 + (2 if with_alpha else 0)


def _groups(bits, groups):
    return list(groups) if groups else [32] * len(bits)


def call_bytes(D, bits, policy, r, G=0, groups=None):
    """Algorithmic HBM bytes one decode call of loop r reads per (b, h, cached token):
    the stored components the reconstruction needs, K and V (fp16 meta and alpha).
    Loops form groups of G (0: one group) with an anchor each; `groups` gives each
    loop's channel group size (default 32)."""
    G = G or len(bits)
    gs = _groups(bits, groups)
    g0 = r // G * G
    if policy == "last":
        a = g0 + G - 1
        comps = [a] if r == a else [a, r]
    else:
        a = g0
        comps = list(range(g0, r + 1))
    return 2 * sum(comp_bytes(D, bits[c], c != a, gs[c]) for c in comps)


PROFILED_WORKLOAD = "ouro_16k"       # the workload the committed counter summaries cover


def dom_kernel_name(D, bits, G, groups=None, rot16=True):
    """Instance name of the streaming kernel decoding loop 1 (anchor + loop-1 residual);
    a component's nibble is its bit width, plus 8 for groups of 16 channels; the last
    parameter is 1 for rotations stored fp16."""
    G = G or len(bits)
    gs = _groups(bits, groups)
    kind = [b | (8 if g == 16 else 0) for b, g in zip(bits, gs)]
    cb = kind[G - 1] | (kind[0] << 4)
    return f"decode_fused<{D}, 2, {cb}u, 2, 2, {1 if rot16 else 0}>"


DOM_KERNEL = dom_kernel_name(128, [2, 2, 4, 4], 0)
COPY_KERNEL = "bitwise_not"
COPY_KIB = float(1 << 20)            # 1 GiB read and 1 GiB written by the calibration kernel
PROFILES = os.path.join(ROOT, "profiles")
FETCH_FILE = os.path.join(PROFILES, "decode_fused_loop1_ouro_16k_fetch_size.txt")
WRITE_FILE = os.path.join(PROFILES, "decode_fused_loop1_ouro_16k_write_size.txt")
KERNEL_SOURCES = ["rq_decode.hip", "rq_decode_kernel.hpp", "rq_combine.hpp", "rq_device.hpp", "rq_internal.hpp"]


def kernel_source_hash():
    """sha256 over the sources of the decode kernels and the build flags."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "decode_attention_quantize_amd")
    for name in KERNEL_SOURCES:
        with open(os.path.join(pkg, "csrc", name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _read_counter_summary(path, counter):
    """(source hash, {kernel: mean KiB per dispatch}) from a summary this script wrote."""
    if not os.path.exists(path):
        return None, {}
    src, vals = None, {}
    with open(path) as f:
        for line in f:
            if line.startswith("# kernel sources sha256:"):
                src = line.split(":", 1)[1].strip()
            elif line.startswith("counter\t" + counter + "\t"):
                _, _, kern, n, mean = line.rstrip("\n").split("\t")
                vals[kern] = float(mean)
    return src, vals


def profiled_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed FETCH_SIZE and
    WRITE_SIZE summaries, each scaled by the copy kernel's reading of its known size;
    None for another workload, or when a summary is missing or was taken on other
    kernel sources."""
    if workload != PROFILED_WORKLOAD:
        return None
    cur = kernel_source_hash()
    total, used = 0.0, []
    for path, counter in ((FETCH_FILE, "FETCH_SIZE"), (WRITE_FILE, "WRITE_SIZE")):
        src, vals = _read_counter_summary(path, counter)
        if src != cur or DOM_KERNEL not in vals:
            return None
        copy = [v for k, v in vals.items() if COPY_KERNEL in k]
        if not copy or copy[0] <= 0:
            return None
        factor = COPY_KIB / copy[0]
        total += vals[DOM_KERNEL] * factor * 1024.0
        used.append(f"{os.path.basename(path)} (x{factor:.4f})")
    return {"bytes": total, "source": ", ".join(used)}


def summarize_profile(directory, title, command):
    """Text summary of rocprofv3 CSV output under `directory`: per-kernel kernel-trace
    statistics, or per-kernel mean counter values (KiB per dispatch for FETCH_SIZE /
    WRITE_SIZE), with the command that made it and the kernel-source hash."""
    import csv
    import glob
    import re

    def short(name):
        m = re.search(r"((?:decode_fused|decode_fused_paged|bf16_fused|combine_kernel|"
                      r"append_kernel|append_unit|prefill_attn_kernel|prefill_vt_kernel)<[^>]*>)", name)
        if m:
            return m.group(1)
        if "read_slots" in name:
            return "read_slots (read-rate calibration, librq_calib.so)"
        if COPY_KERNEL in name:
            return "elementwise " + COPY_KERNEL + " (1 GiB in, 1 GiB out)"
        return "torch/runtime: " + re.sub(r"\s+", " ", name)[:60]

    lines = [f"# {title}", f"# command: {command}", f"# kernel sources sha256: {kernel_source_hash()}"]
    stats = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    counters = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if stats:
        agg = {}
        for row in csv.DictReader(open(stats[0])):
            k = short(row["Name"])
            n, tot = int(row["Calls"]), float(row["TotalDurationNs"])
            a = agg.setdefault(k, [0, 0.0, float("inf"), 0.0])
            a[0] += n
            a[1] += tot
            a[2] = min(a[2], float(row["MinNs"]))
            a[3] = max(a[3], float(row["MaxNs"]))
        total = sum(a[1] for a in agg.values())
        lines.append("kernel\tcalls\tavg_us\tmin_us\tmax_us\ttotal_ms\tpct")
        for k, (n, tot, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            lines.append(f"{k}\t{n}\t{tot / n / 1e3:.2f}\t{mn / 1e3:.2f}\t{mx / 1e3:.2f}\t{tot / 1e6:.2f}\t"
                         f"{100 * tot / total:.1f}")
    for path in counters:
        per = {}
        for row in csv.DictReader(open(path)):
            k = short(row["Kernel_Name"])
            key = (row["Counter_Name"], k)
            d = per.setdefault(key, {})
            did = row["Dispatch_Id"]
            d[did] = d.get(did, 0.0) + float(row["Counter_Value"])
        lines.append("counter\tname\tkernel\tdispatches\tmean_per_dispatch")
        for (cn, k), d in sorted(per.items()):
            if k.startswith("torch/runtime"):
                continue
            lines.append(f"counter\t{cn}\t{k}\t{len(d)}\t{sum(d.values()) / len(d):.1f}")
    return "\n".join(lines) + "\n"


def measure(w, K, warmup, BS=0, want_rq=True, want_chained=True, want_bf16=True, want_percall=False,
            call_reps=50, rot16=True, want_rot32=False):
    """Build workload w's caches (untimed) and time K decode steps of the enabled
    paths, each step captured as one HIP graph. Returns a dict of timings; every
    device buffer is released when it returns."""
    import torch

    import decode_attention_quantize_amd as rq
    import synth

    B, H, D, L, T = w.batch, w.heads, w.D, w.L, w.T
    T_max = T + max(K, warmup)
    if BS:
        T_max = -(-T_max // BS) * BS
    dev = "cuda"
    scale = 1.0 / math.sqrt(D)
    bits, cbits = list(w.bits), list(w.chained_bits)
    G = w.loop_group
    gr, cgr = w.groups_for(bits), w.groups_for(cbits)
    t_build = time.time()
    table, nblocks = None, 0
    if BS:
        # a serving engine's block table: every sequence's blocks scattered over one pool
        nblocks = B * (T_max // BS)
        perm = torch.randperm(nblocks, generator=torch.Generator().manual_seed(1234)).to(torch.int32)
        table = perm.view(B, T_max // BS).to(dev)
    # rotations stored fp16 (as the pages keep the calibrated matrices) or fp32
    rflag = rq.FLAG_ROT_F16 if rot16 else 0
    d_rq = rq.make_desc(B, H, D, bits, T_max, rq.POLICY_LAST_LOOP, group=gr, loop_group=G, block_size=BS,
                        num_blocks=nblocks, flags=rflag)
    d_ch = rq.make_desc(B, H, D, cbits, T_max, rq.POLICY_PREV_LOOP, group=cgr, loop_group=G, block_size=BS,
                        num_blocks=nblocks, flags=rflag)
    # the chained comparator runs where the library has a kernel for every loop's chain
    chain_ok = all(rq.check_decode(d_ch, r) == 0 for r in range(L))
    run_chained = want_chained and chain_ok
    caches, chained, bf16 = [], [], []
    # the BF16 caches of all layers in one tensor, so that one index copy stores a
    # step's current K/V of every layer
    bf16_all = torch.empty(w.layers, 2, L, B, H, T_max, D, dtype=torch.bfloat16, device=dev) if want_bf16 else None
    kvcur = torch.empty(K, w.layers, 2, L, B, H, 1, D, dtype=torch.bfloat16, device=dev)
    qs = torch.empty(K, w.layers, L, B, H, D, dtype=torch.bfloat16, device=dev)
    pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
    n_cur = T_max - T
    for l in range(w.layers):
        # the prompt [0, T) and the decode steps' tokens [T, T_max), generated apart
        # (the generator is seeded per 256-token chunk, so the values are those of one
        # draw over [0, T_max)) to halve the temporary memory at the capacity shape
        past = synth.kv(w, l, 0, T, device=dev)                       # [2][L][B][H][T][D]
        cur = synth.kv(w, l, T, n_cur, device=dev)
        rk, rv = synth.rotation(w, l, 0), synth.rotation(w, l, 1)
        if want_rq:
            c = rq.LayerCache.allocate(d_rq, rk, rv, block_table=table)
            rq.quantize_append(c, past, pos0, T)
            caches.append(c)
        if run_chained:
            cc = rq.LayerCache.allocate(d_ch, rk, rv, block_table=table)
            rq.quantize_append(cc, past, pos0, T)
            chained.append(cc)
        for k in range(K):
            kvcur[k, l] = cur[..., k:k + 1, :]
            for r in range(L):
                qs[k, l, r] = synth.query(w, l, r, k, device=dev)
        if want_bf16:
            bf16_all[l][..., :T, :].copy_(past)
            bf16_all[l][..., T:, :].copy_(cur)
            bf16.append(bf16_all[l])
        del past, cur
        torch.cuda.synchronize()
        if l % 6 == 5 or l == w.layers - 1:
            log(f"{w.name} B{B}: built layer {l + 1}/{w.layers} ({time.time() - t_build:.1f}s)")
    ws = rq.alloc_workspace(d_rq)
    ws_ch = rq.alloc_workspace(d_ch)
    out = torch.empty(w.layers, L, B, H, D, dtype=torch.float32, device=dev)
    past_len = torch.full((B,), T, dtype=torch.int32, device=dev)
    log(f"{w.name} B{B}: caches built: RQ {sum(c.nbytes() for c in caches) / 1e9:.2f} GB, BF16 "
        f"{sum(x.numel() * 2 for x in bf16) / 1e9:.2f} GB, {time.time() - t_build:.1f}s")

    # One step, in the order a looped decoder runs it: for each loop r and layer
    # l, the attention call (streaming launch + combine) that the next layer's
    # query would depend on; after the final loop, the append of the current
    # token to every layer's cache (one call, shared launches); then
    # past_len += 1. All on one stream.
    def rq_step(k, cs, workspace):
        for r in range(L):
            for l in range(w.layers):
                kc = kvcur[k, l, 0, r, :, :, 0]
                vc = kvcur[k, l, 1, r, :, :, 0]
                rq.decode_attn(cs[l], r, qs[k, l, r], kc, vc, past_len, scale, out[l, r], workspace)
        rq.quantize_append_layers(cs, kvcur[k], past_len, 1)
        past_len.add_(1)

    # The BF16 comparator's step pays for its cache store as the RQ step pays for
    # its append: after the final loop, every layer's current K/V of every loop is
    # written at position past_len (one torch index copy over all layers; same
    # values as the prefilled rows, so the attention reads are unchanged).
    bf16_pos = torch.empty(1, dtype=torch.long, device=dev)

    def bf16_step(k):
        bf16_pos.copy_(past_len[:1])
        for r in range(L):
            for l in range(w.layers):
                kc = kvcur[k, l, 0, r, :, :, 0]
                vc = kvcur[k, l, 1, r, :, :, 0]
                rq.decode_attn_bf16(d_rq, bf16[l][0, r], bf16[l][1, r], qs[k, l, r], kc, vc, past_len, scale,
                                    out[l, r], ws)
        bf16_all.index_copy_(5, bf16_pos, kvcur[k])
        past_len.add_(1)

    side = torch.cuda.Stream()

    def capture(fn):
        graphs = []
        torch.cuda.synchronize()
        for k in range(K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn(k)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    def run(graphs):
        for k in range(min(warmup, K)):
            graphs[k].replay()
        torch.cuda.synchronize()
        past_len.fill_(T)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        past_len.fill_(T)
        torch.cuda.synchronize()
        return dt

    mean_ctx = T + (K - 1) / 2.0
    res = {"w": w, "K": K, "mean_ctx": mean_ctx}
    if want_rq:
        log(f"{w.name} B{B}: capturing RQ steps")
        g_rq = capture(lambda k: rq_step(k, caches, ws))
        res["rq_s"] = run(g_rq)
        del g_rq
        res["rq_bytes"] = sum(call_bytes(D, bits, "last", r, G, gr) for r in range(L)) * H * w.layers * B * mean_ctx
        log(f"{w.name} B{B}: RQ {K} steps in {res['rq_s'] * 1e3:.2f} ms")
    caches32 = []
    if want_rq and rot16 and want_rot32:
        # The same caches with fp32 copies of the fp16 rotations (no RQ_FLAG_ROT_F16):
        # bit-identical outputs and stores, so only the rotation reads differ.
        d32 = rq.Desc.from_buffer_copy(d_rq)
        d32.flags = d_rq.flags & ~rq.FLAG_ROT_F16
        caches32 = [rq.LayerCache(d32, c.codes, c.meta, c.alpha, [c.rot[0].float(), c.rot[1].float()],
                                  c.block_table) for c in caches]
        log(f"{w.name} B{B}: capturing RQ steps with fp32 rotations")
        g_32 = capture(lambda k: rq_step(k, caches32, ws))
        res["rq32_s"] = run(g_32)
        del g_32
        log(f"{w.name} B{B}: RQ (fp32 rotations) {K} steps in {res['rq32_s'] * 1e3:.2f} ms")
    if want_chained and not chain_ok:
        res["chained_skipped"] = (f"no decode kernel for every loop of the chained plan {cbits} "
                                  f"(groups {cgr}, loop group {G or L}; see rq_check_decode)")
    elif run_chained:
        log(f"{w.name} B{B}: capturing chained steps")
        g_ch = capture(lambda k: rq_step(k, chained, ws_ch))
        res["ch_s"] = run(g_ch)
        del g_ch
        res["ch_bytes"] = sum(call_bytes(D, cbits, "prev", r, G, cgr) for r in range(L)) * H * w.layers * B * mean_ctx
        log(f"{w.name} B{B}: chained {K} steps in {res['ch_s'] * 1e3:.2f} ms")
    if want_bf16:
        log(f"{w.name} B{B}: capturing BF16 steps")
        g_bf = capture(bf16_step)
        res["bf_s"] = run(g_bf)
        del g_bf
        res["bf_bytes"] = 2 * L * D * 2 * H * w.layers * B * mean_ctx
        log(f"{w.name} B{B}: bf16 {K} steps in {res['bf_s'] * 1e3:.2f} ms")

    if want_percall and want_rq:
        # The streaming kernel (rq_decode_attn_partial's single launch) of each loop
        # of the first group is timed alone: `call_reps` launches (cycling over the
        # layers' caches) captured in a graph, as the steps are, and replayed between
        # two HIP events on the stream the graph is launched on. The combine launch
        # and whole calls are timed the same way.
        stream = torch.cuda.current_stream()

        def events(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(call_reps):
                    fn(i)
            for _ in range(3):               # warm the clocks after the host-side capture
                g.replay()
            torch.cuda.synchronize()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1) / call_reps)
            del g
            return sorted(times)[2]          # median of five replays

        percall = {}
        for r in range(G or L):                       # every loop group has the same shape
            kc = kvcur[0, 0, 0, r, :, :, 0]
            vc = kvcur[0, 0, 1, r, :, :, 0]
            nbytes = call_bytes(D, bits, "last", r, G, gr) * B * H * T
            ms_k = events(lambda i: rq.decode_attn_partial(caches[i % w.layers], r, qs[0, 0, r], past_len, scale,
                                                           ws))
            ms_c = events(lambda i: rq.decode_combine(d_rq, caches[i % w.layers].rot[1], qs[0, 0, r], kc, vc,
                                                      past_len, scale, out[0, r], ws))
            ms_call = events(lambda i: rq.decode_attn(caches[i % w.layers], r, qs[0, 0, r], kc, vc, past_len, scale,
                                                      out[0, r], ws))
            entry = {"kernel_ms": ms_k, "combine_ms": ms_c, "call_ms": ms_call, "bytes": nbytes,
                     "kernel_gbps": nbytes / (ms_k * 1e-3) / 1e9}
            if r == 0:
                # the same launch with the 21-bit rotated query (RQ_FLAG_PRECISE_QUERY)
                ms_p = events(lambda i: rq.decode_attn_partial(caches[i % w.layers], r, qs[0, 0, r], past_len,
                                                               scale, ws, flags=rq.FLAG_PRECISE_QUERY))
                entry["precise_query_kernel_ms"] = ms_p
                if caches32:
                    entry["rot_fp32_kernel_ms"] = events(lambda i: rq.decode_attn_partial(
                        caches32[i % w.layers], r, qs[0, 0, r], past_len, scale, ws))
                entry["read_ceiling"] = read_ceiling(caches, d_rq, r, G or L, bits, gr, T, events, ms_k)
            percall[r] = entry
        res["percall"] = percall
    del caches, caches32, chained, bf16, bf16_all, kvcur, qs, ws, ws_ch, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def _calib_lib():
    """librq_calib.so (the read-rate calibration kernel, built beside librq.so), or None."""
    import ctypes
    path = os.path.join(ROOT, "decode_attention_quantize_amd", "librq_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.rqc_read_slots.restype = ctypes.c_int
    lib.rqc_read_slots.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int)] + \
        [ctypes.c_int] * 7 + [ctypes.c_void_p, ctypes.c_void_p]
    return lib


def read_ceiling(caches, d, r, G, bits, gr, T, events, kernel_ms):
    """The practical read ceiling of loop r's decode traffic: a plain streaming read
    (rqc_read_slots: non-temporal 16-byte loads, no arithmetic) of exactly the
    buffers and per-(b, h) slot ranges the decode call reads, with the same
    workgroup count, timed like the kernel (graphs of launches cycling over the
    layers' caches). Contiguous caches, loops in groups of G, Last-loop."""
    import ctypes
    import torch
    import decode_attention_quantize_amd as rq
    lib = _calib_lib()
    if lib is None:
        log("read ceiling: librq_calib.so not built")
        return None
    if d.block_size or T % 8:
        return None
    unit, nsplit = rq.split_plan(d)
    a = r // G * G + G - 1
    comps = [a] if r == a else [a, r]
    D, B, H = d.head_dim, d.batch, d.heads
    arrays = []
    for c in caches:
        ptrs, bpt = [], []
        for kv in range(2):
            for comp in comps:
                ptrs.append(c.codes[kv][comp].data_ptr())
                bpt.append(D * bits[comp] // 8)
                ptrs.append(c.meta[kv][comp].data_ptr())
                bpt.append(D // gr[comp] * 4)
                if comp != a:
                    ptrs.append(c.alpha[kv][comp].data_ptr())
                    bpt.append(2)
        arrays.append(((ctypes.c_void_p * len(ptrs))(*ptrs), (ctypes.c_int * len(bpt))(*bpt), len(ptrs)))
    row = sum(bpt)
    sink = torch.empty(nsplit * B * H, dtype=torch.int32, device="cuda")

    def launch(i):
        p, b, n = arrays[i % len(arrays)]
        st = lib.rqc_read_slots(p, b, n, B, H, d.max_tokens, T, nsplit, unit, ctypes.c_void_p(sink.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"rqc_read_slots failed ({st})")

    ms = events(launch)
    nbytes = row * B * H * T
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"read ceiling of loop {r + 1}'s traffic: {ms * 1e3:.1f} us, {gbps:.0f} GB/s; kernel/ceiling "
        f"{kernel_ms / ms:.3f}")
    return {"kernel": "read_slots (librq_calib.so): plain non-temporal reads of the call's buffers and slots, same "
                      "workgroup count, no arithmetic",
            "ms_per_launch": ms, "bytes_per_launch": nbytes, "gbps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS,
            "decode_kernel_over_ceiling_time": kernel_ms / ms}


def sub_record(res, label):
    """Compact record of one workload's measure(): tokens/s, the step's algorithmic
    HBM rate and fraction of peak, and the comparators."""
    w, K = res["w"], res["K"]
    rec = {"workload": w.name, "label": label, "layers": w.layers, "batch": w.batch, "heads": w.heads,
           "head_dim": w.D, "loops": w.L, "loop_group": w.loop_group or w.L, "context": w.T, "bits": list(w.bits),
           "steps": K}
    if "rq_s" in res:
        t = res["rq_s"] / K
        rec.update({"value": w.batch * K / res["rq_s"], "unit": "tokens/s", "ms_per_step": t * 1e3,
                    "hbm_gbps_step": res["rq_bytes"] / t / 1e9, "hbm_frac_step": res["rq_bytes"] / t / 1e9 / HBM_PEAK_GBPS})
    if "ch_s" in res:
        rec["chained"] = {"value": w.batch * K / res["ch_s"], "ms_per_step": res["ch_s"] / K * 1e3,
                          "rq_speedup_over_chained": res["ch_s"] / res["rq_s"]}
    if "chained_skipped" in res:
        rec["chained"] = {"skipped": res["chained_skipped"]}
    if "bf_s" in res:
        t = res["bf_s"] / K
        rec["bf16"] = {"value": w.batch * K / res["bf_s"], "ms_per_step": t * 1e3,
                       "hbm_frac_step": res["bf_bytes"] / t / 1e9 / HBM_PEAK_GBPS}
        if "rq_s" in res:
            rec["bf16"]["rq_speedup_over_bf16"] = res["bf_s"] / res["rq_s"]
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="ouro_16k")
    ap.add_argument("--layers", type=int, default=0, help="override layer count (0: workload's)")
    ap.add_argument("--batch", type=int, default=0, help="override batch (0: workload's)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="paged compressed caches with blocks of this many tokens over a shuffled pool (0: contiguous)")
    ap.add_argument("--rot", choices=("fp16", "fp32"), default="fp16",
                    help="storage of the rotation matrices: fp16 as the pages keep them (App. G), or fp32")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chained", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload shapes (uniform INT2 4k, Huginn-shaped 4k, capacity 8k)")
    ap.add_argument("--config-steps", type=int, default=16, help="decode steps of each other workload shape")
    ap.add_argument("--call-reps", type=int, default=50)
    ap.add_argument("--cpu-sample-units", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum timed CPU-oracle seconds")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB read + 1 GiB write elementwise kernel (counter scaling)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("DIR", "TITLE", "COMMAND"),
                    help="print a text summary of rocprofv3 CSV output in DIR and exit")
    args = ap.parse_args()
    if args.summarize_profile:
        print(summarize_profile(*args.summarize_profile), end="")
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this decode path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is "
              "not supported (multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_quantize_amd as rq
    import synth

    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.layers:
        w = w.with_(layers=args.layers)
    if args.batch:
        w = w.with_(batch=args.batch)
    B, H, D, L, T, K = w.batch, w.heads, w.D, w.L, w.T, args.steps
    BS = args.block_size
    bits = list(w.bits)
    G = w.loop_group
    gr = w.groups_for(bits)

    rot16 = args.rot == "fp16"
    res = measure(w, K, args.warmup, BS, want_rq=True, want_chained=not args.no_chained,
                  want_bf16=not args.no_bf16, want_percall=True, call_reps=args.call_reps, rot16=rot16,
                  want_rot32=True)
    dt_rq = res["rq_s"]
    step_bytes = res["rq_bytes"]
    result = {
        "metric": METRIC, "value": B * K / dt_rq, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": dt_rq * 1e3 / K, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8+fp32", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": B, "heads": H, "head_dim": D, "loops": L,
                   "loop_group": G or L, "context": T, "bits": bits, "group": gr, "block_size": BS,
                   "codes": "int2/int4 + fp16 scale/offset + fp16 alpha",
                   "rotation": ("fp16" if rot16 else "fp32") + " [H][D][D] per layer and tensor",
                   "arith": "keys: int8 dot products with a 14-bit fixed-point rotated query; values: fp32 "
                            "multiply-adds of fp16-exact codes; fp32 softmax and accumulation"},
        "hbm_gbps_step": step_bytes / (dt_rq / K) / 1e9,
        "hbm_frac_step": step_bytes / (dt_rq / K) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
    }
    if "chained_skipped" in res:
        log(f"chained comparator skipped: {res['chained_skipped']}")
        result["chained"] = {"policy": "previous-loop", "skipped": res["chained_skipped"]}
    elif "ch_s" in res:
        dt_ch = res["ch_s"]
        result["chained"] = {"policy": "previous-loop", "bits": list(w.chained_bits), "value": B * K / dt_ch,
                             "unit": "tokens/s", "ms_per_step": dt_ch * 1e3 / K,
                             "hbm_gbps_step": res["ch_bytes"] / (dt_ch / K) / 1e9,
                             "rq_speedup_over_chained": dt_ch / dt_rq}
    if "rq32_s" in res:
        # the same step with the rotations stored fp32 (same values, same outputs)
        dt_32 = res["rq32_s"]
        result["rot_fp32"] = {"value": B * K / dt_32, "unit": "tokens/s", "ms_per_step": dt_32 * 1e3 / K,
                              "loop1_kernel_ms": res["percall"][0].get("rot_fp32_kernel_ms"),
                              "rot_fp16_speedup": dt_32 / dt_rq}
    if "bf_s" in res:
        dt_bf = res["bf_s"]
        result["bf16"] = {"value": B * K / dt_bf, "unit": "tokens/s", "ms_per_step": dt_bf * 1e3 / K,
                          "hbm_gbps_step": res["bf_bytes"] / (dt_bf / K) / 1e9,
                          "rq_speedup_over_bf16": dt_bf / dt_rq}

    percall = res["percall"]
    dom = percall[0]
    traffic = None if BS or not rot16 else profiled_traffic(w.name)
    result["roofline"] = {"bound": "hbm", "achieved": dom["kernel_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": dom["kernel_gbps"] / HBM_PEAK_GBPS,
                          "traffic": None if traffic is None else traffic["bytes"],
                          "kernel": dom_kernel_name(D, bits, G, gr, rot16).replace("fused", "fused_paged" if BS else "fused")
                                    + " (rq_decode_attn_partial, loop 1: "
                                    f"INT{bits[(G or L) - 1]} anchor + INT{bits[0]} residual, K and V)",
                          "bytes_per_launch": dom["bytes"], "ms_per_launch": dom["kernel_ms"],
                          "traffic_source": None if traffic is None else traffic["source"]}
    ceiling = dom.pop("read_ceiling", None)
    if ceiling:
        # context for the roofline: the same bytes, slots and grid with no arithmetic
        result["read_ceiling"] = ceiling
    result["per_call"] = {f"loop{r + 1}": v for r, v in percall.items()}

    # ---------------------------------------------------------------- prefill attention
    # rq_prefill_attn over the workload's prompt (B x H x T tokens, one loop): the
    # step that precedes decode (§4.2 "Prefill"). Algorithmic flops: 2 D per
    # (query, visible key) for the scores and 2 D for the value sum, T (T + 1) / 2
    # visible pairs per (b, h) under the causal mask. The bulk store of the prompt
    # after the final loop (rq_quantize_append of T tokens, one layer) is timed
    # beside it against the fp64 matrix-core peak (algorithmic flops: 2 D^2 per
    # rotated row, 2 L B H T rows).
    dev = "cuda"
    stream = torch.cuda.current_stream()
    if not args.no_prefill:
        g = torch.Generator(device=dev).manual_seed(7)
        pq = torch.randn(B, H, T, D, generator=g, device=dev).to(torch.bfloat16)
        Xp = synth.kv(w, 0, 0, T, device=dev)
        pk, pv = Xp[0, 0].contiguous(), Xp[1, 0].contiguous()
        pout = torch.empty(B, H, T, D, dtype=torch.float32, device=dev)
        plens = torch.full((B,), T, dtype=torch.int32, device=dev)
        d_p = rq.make_desc(B, H, D, bits, T, rq.POLICY_LAST_LOOP, group=gr, loop_group=G,
                           flags=rq.FLAG_ROT_F16 if rot16 else 0)
        pws = rq.alloc_prefill_workspace(d_p, T)
        scale = 1.0 / math.sqrt(D)

        def timed(fn, reps=5, warm=2):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            times = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            return sorted(times)[reps // 2]

        ms = timed(lambda: rq.prefill_attn(d_p, pq, pk, pv, plens, scale, pout, pws))
        flops = 4.0 * D * (T * (T + 1) / 2) * B * H
        result["prefill"] = {"kernel": f"prefill_vt_kernel<{D}> + prefill_attn_kernel<{D}> (rq_prefill_attn, "
                                       "one loop, causal; time of both launches)",
                             "tokens": B * T, "ms_per_launch": ms, "flops_per_launch": flops,
                             "tflops": flops / (ms * 1e-3) / 1e12, "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
                             "frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                             "prompt_tokens_per_s": B * T / (ms * 1e-3)}
        log(f"prefill: {ms:.2f} ms per loop-layer, {result['prefill']['tflops']:.0f} TFLOP/s")
        del pq, pk, pv, pout, pws
        cache = rq.LayerCache.allocate(d_p, synth.rotation(w, 0, 0), synth.rotation(w, 0, 1))
        pos0 = torch.zeros(B, dtype=torch.int32, device=dev)
        ms_a = timed(lambda: rq.quantize_append(cache, Xp, pos0, T), reps=3, warm=1)
        aflops = 2.0 * D * D * 2 * L * B * H * T
        result["prompt_store"] = {"kernel": f"append_kernel<{D}> (rq_quantize_append of the {T}-token prompt, one "
                                            "layer, all loops, K and V)",
                                  "ms_per_launch": ms_a, "flops_per_launch": aflops,
                                  "tflops": aflops / (ms_a * 1e-3) / 1e12, "bound": "mfma",
                                  "peak_tflops": FP64_PEAK_TFLOPS, "frac": aflops / (ms_a * 1e-3) / 1e12 / FP64_PEAK_TFLOPS}
        log(f"prompt store: {ms_a:.2f} ms per layer, {result['prompt_store']['tflops']:.1f} TFLOP/s fp64")
        del cache, Xp
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the other workload shapes
    # Uniform INT2 at 4k (B1: fixed per-call costs dominate), the Huginn-shaped
    # recurrence (8 loops in one group, D96, 55 heads) and the 8k capacity shape:
    # RQ at the largest batch the sweep runs (128) against BF16 at the largest
    # batch whose cache fits (32), each with fewer steps than the headline.
    if not args.no_configs and not (args.layers or args.batch or BS):
        cs = args.config_steps
        configs = {}
        for name, label in (("ouro_int2_4k", "uniform INT2, B1, 4k"), ("huginn_4k", "Huginn-shaped, B4, 4k")):
            r = measure(synth.WORKLOADS[name], cs, 2, 0, want_rq=True, want_chained=True, want_bf16=True,
                        rot16=rot16)
            configs[name] = sub_record(r, label)
        cap = synth.WORKLOADS["ouro_8k_capacity"]
        r_rq = measure(cap.with_(batch=128), cs, 2, 0, want_rq=True, want_chained=False, want_bf16=False,
                       rot16=rot16)
        r_bf = measure(cap.with_(batch=32), cs, 2, 0, want_rq=False, want_chained=False, want_bf16=True)
        rec = sub_record(r_rq, "capacity 8k: RQ at batch 128")
        bf = sub_record(r_bf, "capacity 8k: BF16 at batch 32")["bf16"]
        bf["batch"] = 32
        rec["bf16_at_its_largest_batch"] = bf
        rec["rq_peak_over_bf16_peak"] = rec["value"] / bf["value"]
        configs["ouro_8k_capacity"] = rec
        result["configs"] = configs

    if args.calibrate_copy:
        # a plain streaming kernel of known size for scaling the HBM counters:
        # reads 1 GiB and writes 1 GiB
        a = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, bits, args.cpu_sample_units, args.cpu_seconds, torch, synth,
                                              1.0 / math.sqrt(D), rot16)

    print(json.dumps(result), flush=True)


def cpu_baseline(w, bits, units, min_seconds, torch, synth, scale, rot16=True):
    """Time the CPU oracle's decode work on a bounded sample of (b, h) series of
    layer 0 (its own cache, built untimed), scaled to the whole step. The sample
    is repeated until at least min_seconds of wall time have been measured."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle as O

    # every host core this process may run on, within the CPU share the host grants
    # it (OMP_NUM_THREADS where the host sets one)
    visible = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = min(visible, share) if share > 0 else visible
    units = units or w.batch * w.heads
    T, L, D = w.T, w.L, w.D
    pairs = [(u // w.heads % w.batch, u % w.heads) for u in range(units)]
    X = synth.kv(w, 0, 0, T + 1, device="cuda")
    rk, rv = synth.rotation(w, 0, 0), synth.rotation(w, 0, 1)
    if rot16:                                   # the matrices the GPU path stores
        rk, rv = rk.half().float(), rv.half().float()
    rk, rv = rk.numpy(), rv.numpy()
    u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    Xh = {p: u16(X[:, :, p[0], p[1]]) for p in pairs}
    qn = [u16(synth.query(w, 0, r, 0, device="cpu")) for r in range(L)]
    cfg = O.Config(D=D, bits=list(bits), group=w.groups_for(bits), loop_group=w.loop_group)
    t0 = time.time()

    def build(p):
        b, h = p
        return p, (O.quantize_series(cfg, Xh[p][0, :, :T], rk[h], diagnostics=False),
                   O.quantize_series(cfg, Xh[p][1, :, :T], rv[h], diagnostics=False))

    with ThreadPoolExecutor(max_workers=cores) as ex:
        ser = dict(ex.map(build, pairs))
    log(f"cpu baseline: oracle caches for {units} series built in {time.time() - t0:.1f}s")

    def step(p):
        b, h = p
        ks, vs = ser[p]
        for r in range(L):
            O.attend(ks, vs, r, T, rk[h], rv[h], qn[r][b, h], Xh[p][0, r, T], Xh[p][1, r, T], scale)
        O.quantize_series(cfg, Xh[p][0, :, T:T + 1], rk[h], diagnostics=False)
        O.quantize_series(cfg, Xh[p][1, :, T:T + 1], rv[h], diagnostics=False)

    passes, dt = 0, 0.0
    with ThreadPoolExecutor(max_workers=cores) as ex:
        while dt < min_seconds:
            t0 = time.perf_counter()
            list(ex.map(step, pairs))
            dt += time.perf_counter() - t0
            passes += 1
    per_pass = dt / passes
    full = per_pass * (w.batch * w.heads * w.layers) / units
    log(f"cpu baseline: {units} (b,h) series x {L} loops, {passes} passes in {dt:.2f}s on {cores} threads")
    return {"value": w.batch / full, "unit": "tokens/s", "cores": cores, "cores_visible": visible,
            "cores_share": share or None, "kind": "oracle",
            "sample": f"{units} (batch, head) series of layer 0 at {T} cached tokens: all {L} loops of "
                      f"fp64 oracle attention plus one-token quantize-append, on {cores} threads, "
                      f"{passes} passes; per-pass time scaled by {w.batch * w.heads * w.layers}/{units}",
            "sample_seconds": dt}


if __name__ == "__main__":
    main()
