"""Helpers for the GPU parity tests: build caches through the C ABI, build the
oracle's caches from the same bf16 inputs, and compare.

Comparison rules (the oracle is the reference; nothing the HIP path writes is
ever fed to an oracle computation):
  * fp16 metadata (offset o, scale s) and LS coefficients are compared bit for
    bit. A mismatch is exempt only if the oracle's binary64 value before fp16
    rounding lies so close to a rounding breakpoint that a relative
    perturbation of 1e-12 changes its fp16 rounding (the GPU accumulates the
    same binary64 sums in another order).
  * codes are compared bit for bit in groups whose metadata (and LS
    coefficient) matched; an element is exempt when the oracle's (v - o)/s lies
    within 1e-6 of a rounding boundary k + 1/2.
  * every mismatch must be exempt, and exempt elements must stay <= 1e-5 of all.
"""
from __future__ import annotations

import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import decode_attention_quantize_amd as rq
import oracle as O
import synth

REL_BREAK = 1e-12
CODE_DELTA = 1e-6
TOL_ATTN = 2e-3


_LOG_FILE = os.environ.get("RQ_PARITY_LOG")


def log(msg: str):
    """Print a parity record; with RQ_PARITY_LOG set, also append it to that file, so a
    run leaves every logged error and exemption count behind."""
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()
    if _LOG_FILE:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(_LOG_FILE, "a") as f:
            f.write(f"{test}\t{msg}\n")


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def unpack_np(row: np.ndarray, D: int, bits: int, g: int = 32) -> np.ndarray:
    """Test-local unpack of one token's packed codes (layout of include/rq.h)."""
    words = row.view("<u4")
    per = 16 // bits
    half = g // 2
    out = np.zeros(D, np.int64)
    wpg = g * bits // 32
    for e in range(D):
        grp, idx = divmod(e, g)
        h, k = divmod(idx, half)
        j, p = divmod(k, per)
        w = int(words[grp * wpg + j])
        out[e] = (w >> (16 * h + bits * p)) & ((1 << bits) - 1)
    return out


def _ambiguous(pre: float, mode: int) -> bool:
    a = O.f16_encode(np.array([pre * (1 - REL_BREAK), pre * (1 + REL_BREAK)]), mode)
    return a[0] != a[1]


def oracle_series_for(X: np.ndarray, H: np.ndarray, bits, policy, loop_group: int = 0, groups=32) -> O.Series:
    groups = list(groups) if isinstance(groups, (list, tuple)) else groups
    cfg = O.Config(D=X.shape[-1], bits=list(bits), group=groups, policy=policy, loop_group=loop_group)
    return O.quantize_series(cfg, X, H, diagnostics=True)


def oracle_layer(Xall: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor, bits, policy, T: int,
                 units=None, threads: int = 16, loop_group: int = 0, groups=32):
    """Oracle caches for (kv, b, h) series of tokens [0, T). Xall: bf16 [2][L][B][H][>=T][D]."""
    X = Xall[..., :T, :]
    _, L, B, H, _, D = X.shape
    units = units if units is not None else [(b, h) for b in range(B) for h in range(H)]
    Xc = {(b, h): u16(X[:, :, b, h]) for (b, h) in units}
    Hk, Hv = rot_k.cpu().numpy(), rot_v.cpu().numpy()
    jobs = [(kv, b, h) for (b, h) in units for kv in range(2)]

    def run(job):
        kv, b, h = job
        return job, oracle_series_for(Xc[(b, h)][kv], (Hk if kv == 0 else Hv)[h], bits, policy, loop_group,
                                      groups)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(run, jobs))


def logical_rows(cache: rq.LayerCache, pool: np.ndarray) -> np.ndarray:
    """A paged pool [NB][H][BS][...] gathered into logical order [B][H][T_max][...]
    through the block table (rq.h); tokens whose entry is not a valid block are zero."""
    d = cache.desc
    BS, NB = d.block_size, d.num_blocks
    table = cache.block_table.cpu().numpy()                       # [B][T_max / BS]
    t = np.arange(d.max_tokens)
    blk = table[:, t // BS]                                       # [B][T_max]
    ok = (blk >= 0) & (blk < NB)
    g = pool[np.where(ok, blk, 0), :, (t % BS)[None, :]]          # [B][T_max][H][...]
    g = np.where(ok.reshape(ok.shape + (1,) * (g.ndim - 2)), g, 0)
    return np.ascontiguousarray(np.swapaxes(g, 1, 2))


def host_copy(cache: rq.LayerCache) -> dict:
    """Host copies of every cache buffer in logical order [B][H][T_max][...]:
    {(kv, loop): (codes, meta, alpha)}."""
    d = cache.desc
    view = (lambda a: logical_rows(cache, a)) if d.block_size else (lambda a: a)
    return {(kv, r): (view(cache.codes[kv][r].cpu().numpy()), view(u16(cache.meta[kv][r])),
                      None if cache.alpha[kv][r] is None else view(u16(cache.alpha[kv][r])))
            for kv in range(2) for r in range(d.loops)}


def compare_cache(cache: rq.LayerCache, series: dict, T: int, host: dict | None = None) -> dict:
    d = cache.desc
    L, D = d.loops, d.head_dim
    stats = dict(elements=0, exempt_elements=0, meta_exempt=0, alpha_exempt=0, bad=[])
    if host is None:
        host = host_copy(cache)
    for (kv, b, h), s in series.items():
        for r in range(L):
            gc, gm, ga = host[(kv, r)]
            bits, g = d.bits[r], d.group[r]
            skip_tok = np.zeros(T, bool)
            if r != rq.anchor_of(d, r):
                oa = s.alpha[r][:T]
                ga_ = ga[b, h, :T]
                for t in np.nonzero(oa != ga_)[0]:
                    if _ambiguous(s.alpha_pre[r, t], O.RNE):
                        stats["alpha_exempt"] += 1
                        skip_tok[t] = True
                    else:
                        stats["bad"].append(("alpha", kv, b, h, r, int(t), int(oa[t]), int(ga_[t])))
            om = s.meta[r][:T]
            gmm = gm[b, h, :T]
            meta_bad = om != gmm                      # [T][G][2]
            grp_skip = np.zeros(om.shape[:2], bool)
            for t, j, w in zip(*np.nonzero(meta_bad)):
                if skip_tok[t]:
                    continue
                pre = (s.pre_o if w == 0 else s.pre_s)[r, t, j]
                if _ambiguous(pre, O.RD if w == 0 else O.RU):
                    stats["meta_exempt"] += 1
                    grp_skip[t, j] = True
                else:
                    stats["bad"].append(("meta", kv, b, h, r, int(t), int(j), int(w)))
            oc = s.codes[r][:T]
            gcc = gc[b, h, :T]
            rows = np.nonzero(np.any(oc != gcc, axis=1))[0]
            stats["elements"] += T * D
            stats["exempt_elements"] += int(skip_tok.sum()) * D + int(grp_skip.sum()) * g
            for t in rows:
                if skip_tok[t]:
                    continue
                a = unpack_np(oc[t], D, bits, g)
                gg = unpack_np(gcc[t], D, bits, g)
                for e in np.nonzero(a != gg)[0]:
                    if grp_skip[t, e // g]:
                        continue
                    if s.delta[r, t, e] < CODE_DELTA:
                        stats["exempt_elements"] += 1
                    else:
                        stats["bad"].append(("code", kv, b, h, r, int(t), int(e), int(a[e]), int(gg[e])))
    return stats


def assert_cache_parity(stats: dict, label: str):
    frac = stats["exempt_elements"] / max(stats["elements"], 1)
    log(f"{label}: elements={stats['elements']} exempt={stats['exempt_elements']} (frac {frac:.2e}) "
        f"meta_exempt={stats['meta_exempt']} alpha_exempt={stats['alpha_exempt']} bad={len(stats['bad'])}")
    assert not stats["bad"], f"{label}: {len(stats['bad'])} non-exempt mismatches, first {stats['bad'][:5]}"
    assert frac <= 1e-5, f"{label}: exempt fraction {frac}"


def oracle_attention(series: dict, units, loop: int, T_of_b, rot_k, rot_v, q, kcur, vcur, scale,
                     threads: int = 16) -> dict:
    """Oracle outputs for (b, h) units; q/kcur/vcur: bf16 [B][H][D] torch tensors."""
    Hk, Hv = rot_k.cpu().numpy(), rot_v.cpu().numpy()
    qn, kn, vn = u16(q), u16(kcur), u16(vcur)

    def run(u):
        b, h = u
        return u, O.attend(series[(0, b, h)], series[(1, b, h)], loop, int(T_of_b[b]), Hk[h], Hv[h],
                           qn[b, h], kn[b, h], vn[b, h], scale)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(run, units))


def max_rel_err(gpu_out: torch.Tensor, ref: dict) -> float:
    g = gpu_out.detach().cpu().double().numpy()
    worst = 0.0
    for (b, h), o in ref.items():
        err = np.abs(g[b, h] - o).max() / max(np.abs(o).max(), 1e-30)
        worst = max(worst, err)
    return worst


def build_gpu_layer(X: torch.Tensor, rot_k, rot_v, bits, policy, T_max: int, T: int,
                    steps_of_one: int = 0, pos0=None, chunk: int = 1, loop_group: int = 0,
                    groups=32, paging=None, flags: int = 0, zero: bool = False) -> rq.LayerCache:
    """Fill a GPU cache with tokens [0, T) of X (bf16 [2][L][B][H][*][D] on the GPU): one
    bulk append of the first T - steps_of_one tokens, then appends of `chunk` tokens
    (the last one shorter) until T. paging = (block_size, num_blocks, block table) makes
    it a paged cache; flags go into the descriptor (FLAG_ROT_F16: rotations stored fp16);
    zero=True clears every buffer first (rows never written then compare equal)."""
    _, L, B, H, _, D = X.shape
    bs, nb, table = paging if paging else (0, 0, None)
    d = rq.make_desc(B, H, D, bits, T_max, policy, group=groups, loop_group=loop_group, block_size=bs,
                     num_blocks=nb, flags=flags)
    cache = rq.LayerCache.allocate(d, rot_k, rot_v, block_table=table)
    if zero:
        for kv in range(2):
            for r in range(L):
                for t in (cache.codes[kv][r], cache.meta[kv][r], cache.alpha[kv][r]):
                    if t is not None:
                        t.zero_()
    n0 = T - steps_of_one
    pos = torch.zeros(B, dtype=torch.int32, device="cuda") if pos0 is None else pos0
    if n0 > 0:
        rq.quantize_append(cache, X[..., :n0, :].contiguous(), pos, n0)
    t = max(n0, 0)
    while t < T:
        n = min(chunk, T - t)
        p = torch.full((B,), t, dtype=torch.int32, device="cuda")
        rq.quantize_append(cache, X[..., t:t + n, :].contiguous(), p, n)
        t += n
    torch.cuda.synchronize()
    return cache


def inputs(w, T_total, layer=0, batch=None):
    X = synth.kv(w, layer, 0, T_total, device="cuda", batch=batch)
    rk = synth.rotation(w, layer, 0)
    rv = synth.rotation(w, layer, 1)
    return X, rk, rv


def decode_and_compare(w, X, rk, rv, cache, series, lens, loops, label, batch=None, flags=None):
    B, H, D = X.shape[2], X.shape[3], X.shape[5]
    d = cache.desc
    ws = rq.alloc_workspace(d)
    past = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    worst = 0.0
    for r in loops:
        q = synth.query(w, 0, r, 0, device="cuda", batch=B)
        # current token: position lens[b] of sequence b, loop r
        kc = torch.stack([X[0, r, b, :, lens[b]] for b in range(B)]).contiguous()
        vc = torch.stack([X[1, r, b, :, lens[b]] for b in range(B)]).contiguous()
        out = torch.empty(B, H, D, dtype=torch.float32, device="cuda")
        log(f"{label}: decode loop {r}")
        rq.decode_attn(cache, r, q, kc, vc, past, scale, out, ws, flags=flags)
        torch.cuda.synchronize()
        units = [(b, h) for b in range(B) for h in range(H)]
        ref = oracle_attention(series, units, r, lens, rk, rv, q, kc, vc, scale)
        err = max_rel_err(out, ref)
        worst = max(worst, err)
        log(f"{label}: loop {r} max rel err {err:.3e}")
        assert err <= TOL_ATTN, (label, r, err)
    return worst


def shuffled_table(B: int, T_max: int, BS: int, lens, extra: int = 3, seed: int = 0):
    """A block table that scatters every sequence's blocks over a pool with `extra`
    unused blocks, in a seeded random order; entries past ceil(lens[b] / BS) are -1
    (never read). Returns (num_blocks, int32 table [B][T_max / BS] on the GPU)."""
    nbt = T_max // BS
    need = [-(-n // BS) for n in lens]
    nb = sum(need) + extra
    perm = np.random.default_rng(seed).permutation(nb)
    table = np.full((B, nbt), -1, np.int32)
    k = 0
    for b in range(B):
        table[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    return nb, torch.from_numpy(table).cuda()
