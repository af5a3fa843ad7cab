"""Seeded synthetic inputs for the looped-KV decode workloads.

This module only draws random inputs; it contains none of the quantization or
attention arithmetic. Both the CPU oracle (tests) and the HIP path (tests,
benchmark) consume exactly the bf16 tensors it returns.

Input law (per layer and head), standing in for real Ouro-1.4B / Huginn-3.5B
keys and values, which are not available here:
  * key channel scales c_i = exp(0.5 n_i), n_i ~ N(0,1); `outliers` randomly
    chosen channels get c_i <- 8 c_i; values use c = 1;
  * anchor (last loop L):  X_L[t] = c * z_t, z_t ~ N(0, I);
  * loop r < L:            X_r[t] = s_r X_L[t] + sigma_r c * eps_{r,t};
    Ouro-shaped: s_r = 0.8 + 0.05 r, sigma_r = 0.4 / r;
    Huginn-shaped: s_r = 0.7 + 0.03 r, sigma_r = 0.5 / r;
  * with loop groups of G loops (a workload's loop_group), the same law holds
    inside every group with its own anchor draw (the group's last loop) and r
    counted within the group;
  * queries q ~ N(0, I); all tensors rounded to bf16 (round to nearest even);
  * the current token of decode step k sits at position T + k and follows the
    same law;
  * rotations: per (layer, head, K/V) a Sylvester-Hadamard block / sqrt(nb)
    times a seeded +-1 diagonal, block-diagonal when nb < D, stored fp32.

Randomness comes from torch generators seeded per (workload seed, layer,
tensor kind, 256-token chunk), so any token range can be regenerated alone and
a range drawn on one device is bit-identical wherever it is copied.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

CHUNK = 256


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    heads: int
    D: int
    L: int
    T: int                      # cached tokens before the first decode step
    steps: int                  # decode steps
    bits: tuple                 # per loop, Last-loop policy (anchor last)
    chained_bits: tuple         # per loop, Previous-loop policy (anchor first)
    group: int = 32
    outliers: int = 4
    family: str = "ouro"        # "ouro" or "huginn"
    nb: int = 0                 # Hadamard block size (0 -> D)
    seed: int = 0
    loop_group: int = 0         # loops per anchor group (0 -> all L loops)
    int2_group: int = 32        # group size of the 2-bit loops (16 or 32); 4-bit loops use `group`

    @property
    def G(self) -> int:
        return self.loop_group or self.L

    def groups_for(self, bits) -> list:
        """Group size of every loop of a bit plan."""
        return [self.int2_group if b == 2 else self.group for b in bits]

    @property
    def block(self) -> int:
        return self.nb or self.D

    @property
    def t_max(self) -> int:
        return self.T + self.steps

    def sim(self, r: int) -> float:
        """s_r for 1-based loop r < L."""
        return 0.8 + 0.05 * r if self.family == "ouro" else 0.7 + 0.03 * r

    def noise(self, r: int) -> float:
        return 0.4 / r if self.family == "ouro" else 0.5 / r

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # 1 layer, B1, 2 heads, D64, 4 loops, 256 tokens, [2,2,2,4]
    "tiny": Workload("tiny", 1, 1, 2, 64, 4, 256, 1, (2, 2, 2, 4), (4, 2, 2, 2), outliers=2),
    # Ouro-1.4B-shaped, uniform INT2, B1, 4k context, one decode step
    "ouro_int2_4k": Workload("ouro_int2_4k", 24, 1, 16, 128, 4, 4096, 1, (2, 2, 2, 2), (2, 2, 2, 2)),
    # Ouro-1.4B-shaped fixed batch, 16k context, 64 decode steps, [2,2,4,4]
    "ouro_16k": Workload("ouro_16k", 24, 8, 16, 128, 4, 16384, 64, (2, 2, 4, 4), (4, 4, 2, 2)),
    # Ouro-1.4B-shaped capacity sweep at 8k context (batch set per run)
    # the 16k workload with the paper's main mixed plan: INT2 residuals, INT4 anchor only
    "ouro_16k_2224": Workload("ouro_16k_2224", 24, 8, 16, 128, 4, 16384, 64, (2, 2, 2, 4), (4, 2, 2, 2)),
    # the 16k workload with the 2-bit residual loops in groups of 16 channels
    "ouro_16k_g16": Workload("ouro_16k_g16", 24, 8, 16, 128, 4, 16384, 64, (2, 2, 4, 4), (4, 4, 2, 2),
                             int2_group=16),
    "ouro_8k_capacity": Workload("ouro_8k_capacity", 24, 16, 16, 128, 4, 8192, 8, (2, 2, 4, 4), (4, 4, 2, 2)),
    # Huginn-3.5B-shaped: 4 layers, 55 heads, D96 (three 32x32 blocks), 8 recurrences
    "huginn_4k": Workload("huginn_4k", 4, 4, 55, 96, 8, 4096, 1, (2, 2, 2, 2, 2, 2, 4, 4),
                          (4, 4, 2, 2, 2, 2, 2, 2), family="huginn", nb=32),
    # Huginn-3.5B as the paper runs it: 32 recurrences as 8 independent groups of 4, the
    # last loop of each group its anchor (INT4), INT2 residuals
    "huginn32_4k": Workload("huginn32_4k", 4, 4, 55, 96, 32, 4096, 1, (2, 2, 2, 4) * 8, (4, 2, 2, 2) * 8,
                            family="huginn", nb=32, loop_group=4),
}

_KIND = {"kscale": 1, "vscale": 2, "kv": 3, "q": 4, "rot": 5, "outl": 6}


def _gen(w: Workload, layer: int, kind: str, a: int = 0, b: int = 0, device="cpu") -> torch.Generator:
    key = ((((w.seed * 1000003 + layer) * 97 + _KIND[kind]) * 1000033 + a) * 1009 + b) & 0x7FFFFFFFFFFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(key)
    return g


def _hadamard(n: int) -> torch.Tensor:
    W = torch.ones(1, 1, dtype=torch.float64)
    while W.shape[0] < n:
        W = torch.cat([torch.cat([W, W], 1), torch.cat([W, -W], 1)], 0)
    return W


def rotation_signs(w: Workload, layer: int, kv: int) -> torch.Tensor:
    """+-1 int8 [H][D]: the seeded diagonal of each head's rotation."""
    g = _gen(w, layer, "rot", kv)
    return (torch.randint(0, 2, (w.heads, w.D), generator=g, dtype=torch.int64) * 2 - 1).to(torch.int8)


def rotation(w: Workload, layer: int, kv: int, device="cpu") -> torch.Tensor:
    """fp32 [H][D][D], z = H x: block-diag of W_nb / sqrt(nb) times diag(sign)."""
    nb = w.block
    Wb = _hadamard(nb) / math.sqrt(nb)
    blk = torch.block_diag(*([Wb] * (w.D // nb)))
    sign = rotation_signs(w, layer, kv).to(torch.float64)
    H = blk.unsqueeze(0) * sign.unsqueeze(1)          # column j scaled by sign_j
    return H.to(torch.float32).to(device)


def channel_scales(w: Workload, layer: int, device="cpu") -> torch.Tensor:
    """fp32 [H][D] key channel scales with outliers; values use ones."""
    g = _gen(w, layer, "kscale")
    c = torch.exp(0.5 * torch.randn(w.heads, w.D, generator=g, dtype=torch.float32))
    go = _gen(w, layer, "outl")
    for h in range(w.heads):
        idx = torch.randperm(w.D, generator=go)[: w.outliers]
        c[h, idx] *= 8.0
    return c.to(device)


def kv(w: Workload, layer: int, t0: int, n: int, device="cpu", batch=None) -> torch.Tensor:
    """bf16 [2][L][B][H][n][D] for tokens t0 .. t0+n-1 (index 0 = K, 1 = V)."""
    B = w.batch if batch is None else batch
    out = torch.empty(2, w.L, B, w.heads, n, w.D, dtype=torch.bfloat16, device=device)
    ck = channel_scales(w, layer, device).view(1, w.heads, 1, w.D)
    c0, c1 = t0 // CHUNK, (t0 + n - 1) // CHUNK
    for ch in range(c0, c1 + 1):
        lo, hi = max(t0, ch * CHUNK), min(t0 + n, (ch + 1) * CHUNK)
        for t in range(2):
            g = _gen(w, layer, "kv", ch, t, device=device)
            ng, G = w.L // w.G, w.G
            z = torch.randn(ng, B, w.heads, CHUNK, w.D, generator=g, device=device, dtype=torch.float32)
            eps = torch.randn(ng * (G - 1), B, w.heads, CHUNK, w.D, generator=g, device=device,
                              dtype=torch.float32)
            c = ck if t == 0 else torch.ones_like(ck)
            sl = slice(lo - ch * CHUNK, hi - ch * CHUNK)
            o = slice(lo - t0, hi - t0)
            for gi in range(ng):
                anchor = c * z[gi][:, :, sl]
                out[t, gi * G + G - 1, :, :, o] = anchor.to(torch.bfloat16)
                for r in range(1, G):
                    xr = w.sim(r) * anchor + w.noise(r) * c * eps[gi * (G - 1) + r - 1][:, :, sl]
                    out[t, gi * G + r - 1, :, :, o] = xr.to(torch.bfloat16)
    return out


def query(w: Workload, layer: int, loop: int, step: int, device="cpu", batch=None) -> torch.Tensor:
    """bf16 [B][H][D], q ~ N(0, I), for (layer, 0-based loop, decode step)."""
    B = w.batch if batch is None else batch
    g = _gen(w, layer, "q", loop, step, device=device)
    return torch.randn(B, w.heads, w.D, generator=g, device=device).to(torch.bfloat16)


def bits16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
