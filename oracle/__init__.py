"""CPU oracle for the ResidualQuant decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package. The product package never imports it, and this
package imports nothing from the product.

The arithmetic lives in ``rq_oracle.cpp`` (plain binary64 loops, own fp16/bf16
codecs); this module only loads that library with ctypes and marshals numpy
arrays. Citations name the paper page "KV Cache Quantization for Looped
Transformers with 2-Bit Residuals" (ResidualQuant) by section.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(library routines, closed forms, invariants, brute force, the paper's printed
storage numbers). None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rq_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

RNE, RD, RU = 0, 1, 2
LAST_LOOP, PREV_LOOP, FIRST_LOOP = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with g++ (no HIP, no product sources)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


MAX_LOOPS = 32


class _Cfg(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("L", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("loop_group", ctypes.c_int32),
                ("bits", ctypes.c_int32 * MAX_LOOPS), ("group", ctypes.c_int32 * MAX_LOOPS)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.rqo_f16_encode.restype = ctypes.c_uint16
        L.rqo_f16_encode.argtypes = [ctypes.c_double, I]
        L.rqo_f16_decode.restype = ctypes.c_double
        L.rqo_f16_decode.argtypes = [ctypes.c_uint16]
        for n in ("rqo_f16_encode_array",):
            getattr(L, n).argtypes = [P, ctypes.c_int64, I, P]
        for n in ("rqo_f16_decode_array", "rqo_bf16_decode_array"):
            getattr(L, n).argtypes = [P, ctypes.c_int64, P]
        L.rqo_sylvester.argtypes = [I, P]
        L.rqo_rotation.argtypes = [I, I, P, P]
        L.rqo_group_quant.argtypes = [P, I, I, P, P, P, P, P, P]
        L.rqo_group_quant.restype = None
        L.rqo_pack_group.argtypes = [P, I, I, P]
        L.rqo_unpack_group.argtypes = [P, I, I, P]
        L.rqo_row_bytes.argtypes = [P, I]
        L.rqo_quantize_series.argtypes = [P, P, I, P, P, P, P, P, P, P, P]
        L.rqo_reconstruct.argtypes = [P, I, I, P, P, P, P]
        att = [P, I, I, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_double, P]
        L.rqo_attend.argtypes = att
        L.rqo_attend_bruteforce.argtypes = att
        L.rqo_attend_bf16.argtypes = [I, I, P, P, P, P, P, ctypes.c_double, P]
        L.rqo_prefill_attend.argtypes = [I, I, P, P, P, ctypes.c_double, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- formats
def f16_encode(x, mode: int = RNE) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().rqo_f16_encode_array(_p(x), x.size, mode, _p(out))
    return out


def f16_decode(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    lib().rqo_f16_decode_array(_p(h), h.size, _p(out))
    return out


def bf16_decode(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    lib().rqo_bf16_decode_array(_p(h), h.size, _p(out))
    return out


# ---------------------------------------------------------------- rotation
def sylvester(n: int) -> np.ndarray:
    W = np.zeros((n, n), dtype=np.float64)
    if lib().rqo_sylvester(n, _p(W)) != 0:
        raise ValueError("n must be a power of two")
    return W


def rotation(D: int, nb: int, sign) -> np.ndarray:
    sign = np.ascontiguousarray(np.asarray(sign, dtype=np.int8))
    H = np.zeros((D, D), dtype=np.float64)
    if lib().rqo_rotation(D, nb, _p(sign), _p(H)) != 0:
        raise ValueError("nb must be a power of two dividing D")
    return H


# ---------------------------------------------------------------- quantizer
def group_quant(v, bits: int):
    """Returns (o16, s16, codes, delta, pre_o, pre_s) for one group."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    g = v.size
    o = np.zeros(1, np.uint16)
    s = np.zeros(1, np.uint16)
    codes = np.zeros(g, np.uint16)
    delta = np.zeros(g, np.float64)
    po = np.zeros(1, np.float64)
    ps = np.zeros(1, np.float64)
    lib().rqo_group_quant(_p(v), g, bits, _p(o), _p(s), _p(codes), _p(delta), _p(po), _p(ps))
    return int(o[0]), int(s[0]), codes, delta, float(po[0]), float(ps[0])


def pack_group(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint16))
    out = np.zeros(codes.size * bits // 8, np.uint8)
    if lib().rqo_pack_group(_p(codes), codes.size, bits, _p(out)) != 0:
        raise ValueError("unsupported bits/group")
    return out


def unpack_group(data, g: int, bits: int) -> np.ndarray:
    data = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    out = np.zeros(g, np.uint16)
    if lib().rqo_unpack_group(_p(data), g, bits, _p(out)) != 0:
        raise ValueError("unsupported bits/group")
    return out


# ---------------------------------------------------------------- series
@dataclass
class Config:
    D: int
    bits: list
    group: list | int = 32
    policy: int = LAST_LOOP
    loop_group: int = 0                 # loops per anchor group; 0 = all loops one group

    @property
    def L(self) -> int:
        return len(self.bits)

    @property
    def G(self) -> int:
        return self.loop_group or self.L

    def groups(self) -> list:
        return list(self.group) if isinstance(self.group, (list, tuple)) else [self.group] * self.L

    def anchor(self, r: int = 0) -> int:
        """Anchor loop of loop r's group (§3.2, §5 "Models")."""
        g0 = r // self.G * self.G
        return g0 + self.G - 1 if self.policy == LAST_LOOP else g0

    def c(self) -> _Cfg:
        c = _Cfg()
        c.D, c.L, c.policy, c.loop_group = self.D, self.L, self.policy, self.loop_group
        for r, (b, g) in enumerate(zip(self.bits, self.groups())):
            c.bits[r] = b
            c.group[r] = g
        return c

    def row_bytes(self, r: int) -> int:
        return self.D * self.bits[r] // 8

    def n_groups(self, r: int) -> int:
        return self.D // self.groups()[r]


@dataclass
class Series:
    """Packed cache of one (tensor, batch, head) series, one entry per loop."""
    cfg: Config
    T: int
    codes: list                       # [L] uint8 [T][row_bytes]
    meta: list                        # [L] uint16 [T][G][2]
    alpha: list                       # [L] uint16 [T] (anchor: zeros, unused)
    delta: np.ndarray | None = None   # [L][T][D]
    alpha_pre: np.ndarray | None = None
    pre_o: np.ndarray | None = None
    pre_s: np.ndarray | None = None
    _keep: list = field(default_factory=list)

    def ptrs(self):
        L = self.cfg.L
        cp = (ctypes.c_void_p * L)(*[a.ctypes.data for a in self.codes])
        mp = (ctypes.c_void_p * L)(*[a.ctypes.data for a in self.meta])
        ap = (ctypes.c_void_p * L)(*[a.ctypes.data for a in self.alpha])
        self._keep = [cp, mp, ap]
        return cp, mp, ap


def empty_series(cfg: Config, T: int) -> Series:
    L = cfg.L
    return Series(cfg, T,
                  [np.zeros((T, cfg.row_bytes(r)), np.uint8) for r in range(L)],
                  [np.zeros((T, cfg.n_groups(r), 2), np.uint16) for r in range(L)],
                  [np.zeros(T, np.uint16) for _ in range(L)])


def series_from_arrays(cfg: Config, codes, meta, alpha) -> Series:
    """Wrap externally held cache arrays (e.g. slices of a full cache)."""
    T = codes[0].shape[0]
    alpha = [np.ascontiguousarray(a) if a is not None else np.zeros(T, np.uint16) for a in alpha]
    return Series(cfg, T, [np.ascontiguousarray(c) for c in codes],
                  [np.ascontiguousarray(m) for m in meta], alpha)


def quantize_series(cfg: Config, X_bf16: np.ndarray, H32: np.ndarray, diagnostics: bool = True) -> Series:
    """X_bf16: uint16 [L][T][D] (bf16 bit patterns); H32: float32 [D][D] with z = H x."""
    X = np.ascontiguousarray(X_bf16, dtype=np.uint16)
    H = np.ascontiguousarray(H32, dtype=np.float32)
    L, T, D = X.shape
    assert L == cfg.L and D == cfg.D and H.shape == (D, D)
    s = empty_series(cfg, T)
    if diagnostics:
        s.delta = np.zeros((L, T, D))
        s.alpha_pre = np.zeros((L, T))
        s.pre_o = np.zeros((L, T, D))
        s.pre_s = np.zeros((L, T, D))
    cp, mp, ap = s.ptrs()
    nul = ctypes.c_void_p(0)
    rc = lib().rqo_quantize_series(
        ctypes.byref(cfg.c()), _p(X), T, _p(H), cp, mp, ap,
        _p(s.delta) if diagnostics else nul, _p(s.alpha_pre) if diagnostics else nul,
        _p(s.pre_o) if diagnostics else nul, _p(s.pre_s) if diagnostics else nul)
    if rc != 0:
        raise ValueError(f"rqo_quantize_series failed: {rc}")
    return s


def reconstruct(s: Series, r: int, T: int | None = None) -> np.ndarray:
    T = s.T if T is None else T
    out = np.zeros((T, s.cfg.D))
    cp, mp, ap = s.ptrs()
    rc = lib().rqo_reconstruct(ctypes.byref(s.cfg.c()), r, T, cp, mp, ap, _p(out))
    if rc != 0:
        raise ValueError(f"rqo_reconstruct failed: {rc}")
    return out


def _attend(fn, ks: Series, vs: Series, r: int, T: int, HK, HV, q, kcur, vcur, scale: float):
    HK = np.ascontiguousarray(HK, np.float32)
    HV = np.ascontiguousarray(HV, np.float32)
    q = np.ascontiguousarray(q, np.uint16)
    kcur = np.ascontiguousarray(kcur, np.uint16)
    vcur = np.ascontiguousarray(vcur, np.uint16)
    out = np.zeros(ks.cfg.D)
    kc, km, ka = ks.ptrs()
    vc, vm, va = vs.ptrs()
    rc = fn(ctypes.byref(ks.cfg.c()), r, T, kc, km, ka, vc, vm, va, _p(HK), _p(HV),
            _p(q), _p(kcur), _p(vcur), ctypes.c_double(scale), _p(out))
    if rc != 0:
        raise ValueError(f"attention oracle failed: {rc}")
    return out


def attend(ks: Series, vs: Series, r: int, T: int, HK, HV, q, kcur, vcur, scale: float) -> np.ndarray:
    """Fused-path oracle: q' = HK q, scores in the rotated domain, one inverse V rotation."""
    return _attend(lib().rqo_attend, ks, vs, r, T, HK, HV, q, kcur, vcur, scale)


def attend_bruteforce(ks: Series, vs: Series, r: int, T: int, HK, HV, q, kcur, vcur, scale: float) -> np.ndarray:
    return _attend(lib().rqo_attend_bruteforce, ks, vs, r, T, HK, HV, q, kcur, vcur, scale)


def prefill_attend(Q, K, V, scale: float) -> np.ndarray:
    """Causal attention of one loop over its bf16 prompt (§4.2 "Prefill"): Q, K, V uint16
    [T][D] bf16 bit patterns of one (sequence, head); returns fp64 [T][D]."""
    Q = np.ascontiguousarray(Q, np.uint16)
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    T, D = Q.shape
    assert K.shape == (T, D) and V.shape == (T, D)
    out = np.zeros((T, D))
    if lib().rqo_prefill_attend(D, T, _p(Q), _p(K), _p(V), ctypes.c_double(scale), _p(out)) != 0:
        raise ValueError("rqo_prefill_attend failed")
    return out


def attend_bf16(K, V, q, kcur, vcur, scale: float) -> np.ndarray:
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    T, D = K.shape
    out = np.zeros(D)
    rc = lib().rqo_attend_bf16(D, T, _p(K), _p(V), _p(np.ascontiguousarray(q, np.uint16)),
                               _p(np.ascontiguousarray(kcur, np.uint16)),
                               _p(np.ascontiguousarray(vcur, np.uint16)), ctypes.c_double(scale), _p(out))
    if rc != 0:
        raise ValueError("rqo_attend_bf16 failed")
    return out
