"""Python binding of librq, the C-ABI ResidualQuant decode library for MI355X.

Argument marshalling only: every step of the decode path (rotation,
quantization, packing, fused dequantize + attention, combine) runs in the HIP
kernels of ``librq.so``. PyTorch provides device memory and streams.

Importing this package loads ``librq.so`` from the package directory and fails
loudly if it is missing; build it with ``python
decode_attention_quantize_amd/build.py`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librq.so")
MAX_LOOPS = 32

OK = 0
STATUS = {0: "RQ_OK", 1: "RQ_E_NULL", 2: "RQ_E_SHAPE", 3: "RQ_E_BITS", 4: "RQ_E_CAPACITY",
          5: "RQ_E_WORKSPACE", 6: "RQ_E_UNSUPPORTED", 7: "RQ_E_HIP", 8: "RQ_E_POLICY", 9: "RQ_E_LOOP",
          10: "RQ_E_ALIGN", 11: "RQ_E_SCRATCH"}
SCRATCH_BYTES = 8 << 20                  # RQ_SCRATCH_BYTES of rq.h
POLICY_LAST_LOOP, POLICY_PREV_LOOP, POLICY_FIRST_LOOP = 0, 1, 2
DEVERR_CAPACITY, DEVERR_LENGTH, DEVERR_BLOCK, DEVERR_RANGE = 1, 2, 4, 8
FLAG_PRECISE_QUERY = 1
FLAG_ROT_F16 = 2                         # the cache's rotations are stored fp16 (rq.h RQ_FLAG_ROT_F16)


class RQError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_str(code)})")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("loops", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("loop_group", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("flags", ctypes.c_int32),
                ("bits", ctypes.c_uint8 * MAX_LOOPS), ("group", ctypes.c_uint8 * MAX_LOOPS)]


class LayerCacheC(ctypes.Structure):
    _fields_ = [("codes", (ctypes.c_void_p * MAX_LOOPS) * 2), ("meta", (ctypes.c_void_p * MAX_LOOPS) * 2),
                ("alpha", (ctypes.c_void_p * MAX_LOOPS) * 2), ("rot", ctypes.c_void_p * 2),
                ("block_table", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"librq.so not found at {LIB_PATH}; build it first "
                          "(python decode_attention_quantize_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.rq_buffer_bytes.restype = Z
    L.rq_buffer_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
    L.rq_workspace_bytes.restype = Z
    L.rq_workspace_bytes.argtypes = [P]
    L.rq_check_desc.restype = ctypes.c_int
    L.rq_check_desc.argtypes = [P]
    L.rq_check_decode.restype = ctypes.c_int
    L.rq_check_decode.argtypes = [P, ctypes.c_int32]
    L.rq_quantize_append.restype = ctypes.c_int
    L.rq_quantize_append.argtypes = [P, P, P, P, I, P, P]
    L.rq_quantize_append_layers.restype = ctypes.c_int
    L.rq_quantize_append_layers.argtypes = [P, P, I, P, P, I, P, P]
    L.rq_decode_attn.restype = ctypes.c_int
    L.rq_decode_attn.argtypes = [P, P, I, P, P, P, P, ctypes.c_float, P, P, Z, P, P]
    L.rq_decode_attn_noalloc.restype = ctypes.c_int
    L.rq_decode_attn_noalloc.argtypes = [P, P, I, P, P, P, P, ctypes.c_float, P, P, P]
    L.rq_split_plan.restype = ctypes.c_int
    L.rq_split_plan.argtypes = [P, P, P]
    L.rq_decode_attn_partial.restype = ctypes.c_int
    L.rq_decode_attn_partial.argtypes = [P, P, I, P, P, ctypes.c_float, P, Z, P]
    L.rq_decode_combine.restype = ctypes.c_int
    L.rq_decode_combine.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, Z, P, P]
    L.rq_decode_attn_bf16_partial.restype = ctypes.c_int
    L.rq_decode_attn_bf16_partial.argtypes = [P, P, P, P, P, ctypes.c_float, P, Z, P]
    L.rq_decode_attn_bf16.restype = ctypes.c_int
    L.rq_decode_attn_bf16.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, P, P, Z, P, P]
    L.rq_prefill_attn.restype = ctypes.c_int
    L.rq_prefill_attn.argtypes = [P, P, P, P, P, I, ctypes.c_float, P, P, Z, P, P]
    L.rq_prefill_workspace_bytes.restype = Z
    L.rq_prefill_workspace_bytes.argtypes = [P, I]
    L.rq_status_str.restype = ctypes.c_char_p
    L.rq_status_str.argtypes = [ctypes.c_int]
    L.rq_version.restype = ctypes.c_char_p
    L.rq_version.argtypes = []
    return L


lib = _load()


def status_str(code: int) -> str:
    return lib.rq_status_str(code).decode()


def version() -> str:
    return lib.rq_version().decode()


def make_desc(batch: int, heads: int, head_dim: int, bits, max_tokens: int,
              policy: int = POLICY_LAST_LOOP, group=32, loop_group: int = 0, block_size: int = 0,
              num_blocks: int = 0, flags: int = 0) -> Desc:
    """Descriptor of one layer's cache; `group` is one size for all loops or one per loop;
    block_size > 0 makes it a paged cache of num_blocks blocks; flags: FLAG_PRECISE_QUERY,
    FLAG_ROT_F16 (see rq.h)."""
    d = Desc()
    d.batch, d.heads, d.head_dim = batch, heads, head_dim
    d.loops, d.max_tokens, d.policy, d.loop_group = len(bits), max_tokens, policy, loop_group
    d.block_size, d.num_blocks, d.flags = block_size, num_blocks, flags
    groups = list(group) if isinstance(group, (list, tuple)) else [group] * len(bits)
    if len(groups) != len(bits):
        raise ValueError("one group size per loop")
    for r, (b, g) in enumerate(zip(bits, groups)):
        d.bits[r] = b
        d.group[r] = g
    return d


def rot_dtype(d: Desc):
    """dtype of the cache's rotation matrices under d: float16 with FLAG_ROT_F16, else float32."""
    return torch.float16 if d.flags & FLAG_ROT_F16 else torch.float32


def anchor_of(d: Desc, r: int) -> int:
    """Anchor loop of the loop group holding loop r (the rule stated in rq.h)."""
    G = d.loop_group or d.loops
    g0 = r // G * G
    return g0 + G - 1 if d.policy == POLICY_LAST_LOOP else g0


def check_desc(d: Desc) -> int:
    return lib.rq_check_desc(ctypes.byref(d))


def check_decode(d: Desc, loop: int) -> int:
    """0 when a decode kernel exists for `loop` under d (and its flags), else the status."""
    return lib.rq_check_decode(ctypes.byref(d), loop)


def buffer_bytes(d: Desc, kind: int, loop: int) -> int:
    return lib.rq_buffer_bytes(ctypes.byref(d), kind, loop)


def workspace_bytes(d: Desc) -> int:
    return lib.rq_workspace_bytes(ctypes.byref(d))


def split_plan(d: Desc) -> tuple[int, int]:
    """(unit, nsplit): nsplit slots per (b, h); slot length for a sequence of
    `n` cached tokens is slot_len(n, nsplit, unit)."""
    unit, nsplit = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.rq_split_plan(ctypes.byref(d), ctypes.byref(unit), ctypes.byref(nsplit)), "rq_split_plan")
    return unit.value, nsplit.value


def slot_len(n: int, nsplit: int, unit: int) -> int:
    """Tokens per slot for a sequence of n cached tokens (the rule stated in rq.h)."""
    c = -(-n // nsplit)
    c = -(-c // unit) * unit
    return max(c, unit)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if isinstance(stream, int):
        return stream
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class LayerCache:
    """Device buffers of one layer's compressed cache (caller-owned, allocated by torch)."""
    desc: Desc
    codes: list      # [2][L] uint8 tensors [B][H][T_max][D*bits/8]  (paged: [NB][H][BS][..])
    meta: list       # [2][L] int16 tensors [B][H][T_max][D/g][2] (fp16 bit patterns)
    alpha: list      # [2][L] int16 tensors [B][H][T_max] or None for a group's anchor
    rot: list        # [2] [H][D][D], float32 (float16 with FLAG_ROT_F16)
    block_table: torch.Tensor | None = None   # paged: int32 [B][T_max / BS]

    @staticmethod
    def allocate(d: Desc, rot_k: torch.Tensor, rot_v: torch.Tensor, device="cuda",
                 block_table: torch.Tensor | None = None) -> "LayerCache":
        H, D, L = d.heads, d.head_dim, d.loops
        if d.block_size:
            if block_table is None or block_table.dtype != torch.int32:
                raise ValueError("a paged cache needs an int32 block table [B][max_tokens / block_size]")
            lead = (d.num_blocks, H, d.block_size)
        else:
            lead = (d.batch, H, d.max_tokens)
        codes = [[torch.empty(*lead, D * d.bits[r] // 8, dtype=torch.uint8, device=device)
                  for r in range(L)] for _ in range(2)]
        meta = [[torch.empty(*lead, D // d.group[r], 2, dtype=torch.int16, device=device)
                 for r in range(L)] for _ in range(2)]
        alpha = [[None if r == anchor_of(d, r) else torch.empty(*lead, dtype=torch.int16, device=device)
                  for r in range(L)] for _ in range(2)]
        rdt = rot_dtype(d)   # fp16 storage rounds the given matrices to fp16
        rot = [rot_k.to(device=device, dtype=rdt).contiguous(), rot_v.to(device=device, dtype=rdt).contiguous()]
        table = None if not d.block_size else block_table.to(device).contiguous()
        return LayerCache(d, codes, meta, alpha, rot, table)

    def validate(self):
        """Every buffer's size, dtype and layout against the descriptor (once)."""
        if getattr(self, "_valid", False):
            return
        d = self.desc
        if check_desc(d) != OK:
            raise ValueError(f"cache descriptor invalid (status {check_desc(d)})")
        for kv in range(2):
            for r in range(d.loops):
                for kind, t, dt, name in ((0, self.codes[kv][r], torch.uint8, "codes"),
                                          (1, self.meta[kv][r], torch.int16, "meta"),
                                          (2, self.alpha[kv][r], torch.int16, "alpha")):
                    want = buffer_bytes(d, kind, r)
                    if kind == 2 and r == anchor_of(d, r):
                        continue
                    _need(t, None, dt, f"cache {name}[{kv}][{r}]")
                    if t.numel() * t.element_size() != want:
                        raise ValueError(f"cache {name}[{kv}][{r}]: {t.numel() * t.element_size()} bytes, "
                                         f"the descriptor needs {want}")
            _need(self.rot[kv], (d.heads, d.head_dim, d.head_dim), rot_dtype(d), f"cache rot[{kv}]")
        if d.block_size:
            _need(self.block_table, (d.batch, d.max_tokens // d.block_size), torch.int32, "block_table")
        bufs = {f"cache codes[{kv}][{r}]": self.codes[kv][r] for kv in range(2) for r in range(d.loops)}
        bufs.update({f"cache meta[{kv}][{r}]": self.meta[kv][r] for kv in range(2) for r in range(d.loops)})
        bufs.update({f"cache alpha[{kv}][{r}]": self.alpha[kv][r] for kv in range(2) for r in range(d.loops)})
        bufs.update({"cache rot[0]": self.rot[0], "cache rot[1]": self.rot[1], "block_table": self.block_table})
        _on_gpu(**bufs)
        self._valid = True

    def c(self) -> LayerCacheC:
        self.validate()
        c = LayerCacheC()
        for kv in range(2):
            for r in range(self.desc.loops):
                c.codes[kv][r] = _ptr(self.codes[kv][r])
                c.meta[kv][r] = _ptr(self.meta[kv][r])
                c.alpha[kv][r] = _ptr(self.alpha[kv][r])
            c.rot[kv] = _ptr(self.rot[kv])
        c.block_table = _ptr(self.block_table)
        return c

    def nbytes(self) -> int:
        n = 0
        for kv in range(2):
            for r in range(self.desc.loops):
                n += self.codes[kv][r].numel() + 2 * self.meta[kv][r].numel()
                if self.alpha[kv][r] is not None:
                    n += 2 * self.alpha[kv][r].numel()
        return n


def _need(t, shape, dtype, what: str, optional: bool = False):
    """The C ABI takes raw pointers and cannot see sizes: every tensor handed to
    it is checked here, before the call, for its shape, dtype and layout (a wrong
    size would make a kernel read or write past the tensor); _on_gpu then checks
    the devices."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{what}: missing")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")


def _on_gpu(**tensors):
    for what, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{what}: must be on a GPU device")


def _need_err(dev_err):
    if dev_err is not None:
        _need(dev_err, None, torch.int32, "dev_err")
        if dev_err.numel() < 1:
            raise ValueError("dev_err: needs one int32")


def _need_bytes(t, nbytes: int, what: str):
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError(f"{what}: must be a contiguous tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _check(code: int, where: str):
    if code != OK:
        raise RQError(code, where)


def quantize_append(cache: LayerCache, kv: torch.Tensor, pos: torch.Tensor, n: int,
                    dev_err: torch.Tensor | None = None, stream=None):
    """kv: bf16 [2][L][B][H][n][D]; pos: int32 [B] on the device."""
    d = cache.desc
    _need(kv, (2, d.loops, d.batch, d.heads, n, d.head_dim), torch.bfloat16, "kv")
    _need(pos, (d.batch,), torch.int32, "pos")
    _need_err(dev_err)
    _on_gpu(kv=kv, pos=pos, dev_err=dev_err)
    cc = cache.c()
    _check(lib.rq_quantize_append(ctypes.byref(cache.desc), ctypes.byref(cc), _ptr(kv), _ptr(pos), n,
                                  _ptr(dev_err), _stream(stream)), "rq_quantize_append")


def quantize_append_layers(caches: list, kv: torch.Tensor, pos: torch.Tensor, n: int,
                           dev_err: torch.Tensor | None = None, stream=None):
    """quantize_append for several layers in one call (the layers share launches):
    kv bf16 [nlayers][2][L][B][H][n][D], layer l's input at kv[l]; pos int32 [B]."""
    if len(caches) == 0:
        return
    d = caches[0].desc
    for l, c in enumerate(caches):
        if bytes(c.desc) != bytes(d):
            raise ValueError(f"caches[{l}]: descriptor differs from caches[0]")
    _need(kv, (len(caches), 2, d.loops, d.batch, d.heads, n, d.head_dim), torch.bfloat16, "kv")
    _need(pos, (d.batch,), torch.int32, "pos")
    _need_err(dev_err)
    _on_gpu(kv=kv, pos=pos, dev_err=dev_err)
    arr = (LayerCacheC * len(caches))(*[c.c() for c in caches])
    _check(lib.rq_quantize_append_layers(ctypes.byref(d), arr, len(caches), _ptr(kv), _ptr(pos), n,
                                         _ptr(dev_err), _stream(stream)), "rq_quantize_append_layers")


def prefill_workspace_bytes(d: Desc, n: int) -> int:
    return lib.rq_prefill_workspace_bytes(ctypes.byref(d), n)


def alloc_prefill_workspace(d: Desc, n: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(prefill_workspace_bytes(d, n), 1), dtype=torch.uint8, device=device)


def prefill_attn(d: Desc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, scale: float,
                 out: torch.Tensor, workspace: torch.Tensor | None = None, dev_err: torch.Tensor | None = None,
                 stream=None):
    """Causal prefill attention of one loop: q, k, v bf16 [B][H][n][D]; lens int32 [B];
    out fp32 [B][H][n][D] (rows past lens[b] not written). The workspace is allocated
    here when not given."""
    n = q.shape[2] if isinstance(q, torch.Tensor) and q.dim() == 4 else -1
    shape = (d.batch, d.heads, n, d.head_dim)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, shape, torch.bfloat16, name)
    _need(lens, (d.batch,), torch.int32, "lens")
    _need(out, shape, torch.float32, "out")
    _need_err(dev_err)
    if workspace is None:
        workspace = alloc_prefill_workspace(d, n, q.device)
    _need_bytes(workspace, prefill_workspace_bytes(d, n), "workspace")
    _on_gpu(q=q, k=k, v=v, lens=lens, out=out, workspace=workspace, dev_err=dev_err)
    _check(lib.rq_prefill_attn(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(lens), n, scale, _ptr(out),
                               _ptr(workspace), workspace.numel(), _ptr(dev_err), _stream(stream)),
           "rq_prefill_attn")


def _need_step(d: Desc, q, past_len, k_cur=None, v_cur=None, out=None, full=True):
    bhd = (d.batch, d.heads, d.head_dim)
    _need(q, bhd, torch.bfloat16, "q")
    _need(past_len, (d.batch,), torch.int32, "past_len")
    if full:
        _need(k_cur, bhd, torch.bfloat16, "k_cur")
        _need(v_cur, bhd, torch.bfloat16, "v_cur")
        _need(out, bhd, torch.float32, "out")


def _with_flags(d: Desc, flags) -> Desc:
    """The descriptor as passed to a decode call: flags=None keeps the cache's own; the
    rotation storage (FLAG_ROT_F16) is the cache's and is never overridden."""
    if flags is None:
        return d
    flags = (flags & ~FLAG_ROT_F16) | (d.flags & FLAG_ROT_F16)
    if flags == d.flags:
        return d
    c = Desc.from_buffer_copy(d)
    c.flags = flags
    return c


def decode_attn(cache: LayerCache, loop: int, q, k_cur, v_cur, past_len, scale: float, out, workspace,
                dev_err=None, stream=None, flags=None):
    """flags (e.g. FLAG_PRECISE_QUERY) override the cache descriptor's for this call."""
    _need_step(cache.desc, q, past_len, k_cur, v_cur, out)
    _need_err(dev_err)
    _need_bytes(workspace, 1, "workspace")
    _on_gpu(q=q, k_cur=k_cur, v_cur=v_cur, past_len=past_len, out=out, workspace=workspace, dev_err=dev_err)
    cc = cache.c()
    _check(lib.rq_decode_attn(ctypes.byref(_with_flags(cache.desc, flags)), ctypes.byref(cc), loop, _ptr(q), _ptr(k_cur),
                              _ptr(v_cur), _ptr(past_len), scale, _ptr(out), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(dev_err), _stream(stream)),
           "rq_decode_attn")


def decode_attn_noalloc(cache: LayerCache, loop: int, q, k_cur, v_cur, past_len, scale: float, out,
                        dev_err=None, stream=None, flags=None):
    """decode_attn without a workspace: the library's static per-device scratch holds the
    partials (calls on one GPU must not overlap)."""
    _need_step(cache.desc, q, past_len, k_cur, v_cur, out)
    _need_err(dev_err)
    _on_gpu(q=q, k_cur=k_cur, v_cur=v_cur, past_len=past_len, out=out, dev_err=dev_err)
    cc = cache.c()
    _check(lib.rq_decode_attn_noalloc(ctypes.byref(_with_flags(cache.desc, flags)), ctypes.byref(cc), loop, _ptr(q),
                                      _ptr(k_cur), _ptr(v_cur), _ptr(past_len), scale, _ptr(out), _ptr(dev_err),
                                      _stream(stream)), "rq_decode_attn_noalloc")


def decode_attn_partial(cache: LayerCache, loop: int, q, past_len, scale: float, workspace, stream=None,
                        flags=None):
    """First launch of decode_attn: per-slot partials (m, l, -, -, acc[D]) into the workspace."""
    _need_step(cache.desc, q, past_len, full=False)
    _need_bytes(workspace, 1, "workspace")
    _on_gpu(q=q, past_len=past_len, workspace=workspace)
    cc = cache.c()
    _check(lib.rq_decode_attn_partial(ctypes.byref(_with_flags(cache.desc, flags)), ctypes.byref(cc), loop, _ptr(q),
                                      _ptr(past_len),
                                      scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "rq_decode_attn_partial")


def decode_combine(d: Desc, rot_v, q, k_cur, v_cur, past_len, scale: float, out, workspace, dev_err=None,
                   stream=None):
    """Second launch of decode_attn: merge the workspace partials with the current token."""
    _need_step(d, q, past_len, k_cur, v_cur, out)
    _need(rot_v, (d.heads, d.head_dim, d.head_dim), rot_dtype(d), "rot_v", optional=True)
    _need_err(dev_err)
    _need_bytes(workspace, 1, "workspace")
    _on_gpu(rot_v=rot_v, q=q, k_cur=k_cur, v_cur=v_cur, past_len=past_len, out=out, workspace=workspace,
            dev_err=dev_err)
    _check(lib.rq_decode_combine(ctypes.byref(d), _ptr(rot_v), _ptr(q), _ptr(k_cur), _ptr(v_cur), _ptr(past_len),
                                 scale, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(dev_err), _stream(stream)), "rq_decode_combine")


def _need_bf16_cache(d: Desc, k_cache, v_cache):
    shape = (d.batch, d.heads, d.max_tokens, d.head_dim)
    _need(k_cache, shape, torch.bfloat16, "k_cache")
    _need(v_cache, shape, torch.bfloat16, "v_cache")


def decode_attn_bf16(d: Desc, k_cache, v_cache, q, k_cur, v_cur, past_len, scale: float, out, workspace,
                     dev_err=None, stream=None):
    _need_bf16_cache(d, k_cache, v_cache)
    _need_step(d, q, past_len, k_cur, v_cur, out)
    _need_err(dev_err)
    _need_bytes(workspace, 1, "workspace")
    _on_gpu(k_cache=k_cache, v_cache=v_cache, q=q, k_cur=k_cur, v_cur=v_cur, past_len=past_len, out=out,
            workspace=workspace, dev_err=dev_err)
    _check(lib.rq_decode_attn_bf16(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(k_cur),
                                   _ptr(v_cur), _ptr(past_len), scale, _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(dev_err),
                                   _stream(stream)), "rq_decode_attn_bf16")


def decode_attn_bf16_partial(d: Desc, k_cache, v_cache, q, past_len, scale: float, workspace, stream=None):
    """First launch of decode_attn_bf16: per-slot partials into the workspace (original domain)."""
    _need_bf16_cache(d, k_cache, v_cache)
    _need_step(d, q, past_len, full=False)
    _need_bytes(workspace, 1, "workspace")
    _on_gpu(k_cache=k_cache, v_cache=v_cache, q=q, past_len=past_len, workspace=workspace)
    _check(lib.rq_decode_attn_bf16_partial(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(q), _ptr(past_len),
                                           scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)), "rq_decode_attn_bf16_partial")


def alloc_workspace(d: Desc, device="cuda") -> torch.Tensor:
    """Workspace for the decode calls (any initial contents; zero-filled here)."""
    n = workspace_bytes(d)
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
