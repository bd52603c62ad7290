"""Python binding of librlq (ctypes): torch tensors in, C ABI calls out.

This module only marshals arguments; every step of the computation runs in
the HIP kernels of librlq.so.  It raises if the library is missing - there is
no fallback path.  Names and argument meanings follow include/rlq.h.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librlq.so")

RLQ_OK, RLQ_EINVAL, RLQ_EUNSUPPORTED, RLQ_ENOSPC, RLQ_EHIP = 0, -1, -2, -3, -4
DC, DR, GROUP, NGROUPS, PAGE, WORDS = 512, 64, 128, 4, 64, 32

EXPORTED = (
    "rlq_abi_version", "rlq_layer_params_default", "rlq_status_string", "rlq_last_hip_error",
    "rlq_coupled_gain", "rlq_quantize_append", "rlq_mla_decode_workspace_size", "rlq_mla_decode",
    "rlq_mla_extend_workspace_size", "rlq_mla_extend", "rlq_mla_decode_noalloc",
    "rlq_check_decode_tables", "rlq_check_append_tables", "rlq_check_extend_tables",
)
NOALLOC_SCRATCH_BYTES = 64 << 20   # RLQ_NOALLOC_SCRATCH_BYTES


class LayerParams(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("gain", ctypes.c_float),
                ("level_inner", ctypes.c_float), ("level_outer", ctypes.c_float)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("sink", ctypes.c_void_p), ("recent", ctypes.c_void_p),
                ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("max_batch", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librlq.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_attention_rlq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.rlq_abi_version.restype = ctypes.c_int
    L.rlq_abi_version.argtypes = []
    L.rlq_layer_params_default.restype = LayerParams
    L.rlq_layer_params_default.argtypes = []
    L.rlq_status_string.restype = ctypes.c_char_p
    L.rlq_status_string.argtypes = [ctypes.c_int]
    L.rlq_last_hip_error.restype = ctypes.c_char_p
    L.rlq_last_hip_error.argtypes = []
    L.rlq_coupled_gain.restype = f32
    L.rlq_coupled_gain.argtypes = [f32, f32, f32]
    L.rlq_quantize_append.restype = ctypes.c_int
    L.rlq_quantize_append.argtypes = [
        ctypes.POINTER(LayerParams), ctypes.POINTER(CacheDesc), vp, vp, vp, vp, vp, vp, vp,
        i32, i32, i64, vp, vp]
    L.rlq_mla_decode_workspace_size.restype = ctypes.c_int
    L.rlq_mla_decode_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.rlq_mla_decode.restype = ctypes.c_int
    L.rlq_mla_decode.argtypes = [
        ctypes.POINTER(LayerParams), ctypes.POINTER(CacheDesc), vp, vp, i32, i32, f32,
        vp, i32, vp, i32, vp, vp, vp, ctypes.c_size_t, vp]
    L.rlq_mla_decode_noalloc.restype = ctypes.c_int
    L.rlq_mla_decode_noalloc.argtypes = [
        ctypes.POINTER(LayerParams), ctypes.POINTER(CacheDesc), vp, vp, i32, i32, f32,
        vp, i32, vp, i32, vp, vp, vp]
    for name, extra in (("rlq_check_decode_tables", [i32, vp, vp, i32, i32, i32]),
                        ("rlq_check_append_tables", [i32, vp, vp, vp, i32, i32, i64]),
                        ("rlq_check_extend_tables", [i32, vp, vp, vp, i32, i32, i32, i32])):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = extra
    L.rlq_mla_extend_workspace_size.restype = ctypes.c_int
    L.rlq_mla_extend_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.rlq_mla_extend.restype = ctypes.c_int
    L.rlq_mla_extend.argtypes = [
        ctypes.POINTER(LayerParams), ctypes.POINTER(CacheDesc), vp, vp, vp, i32, i32, i32, f32,
        vp, i32, vp, i32, vp, vp, vp, ctypes.c_size_t, vp]
    _lib = L
    return L


class RlqError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().rlq_status_string(status).decode()
        if status == RLQ_EHIP:
            msg += " (" + lib().rlq_last_hip_error().decode() + ")"
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != RLQ_OK:
        if status == RLQ_EINVAL:
            raise ValueError(f"{where}: {lib().rlq_status_string(status).decode()}")
        raise RlqError(status, where)


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None = None, name: str = "") -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t: torch.Tensor | None, shape: tuple, name: str):
    """Raise ValueError unless t has `shape` (None entries match any size)."""
    if t is None:
        return
    ok = t.dim() == len(shape) and all(w is None or int(d) == w for d, w in zip(t.shape, shape))
    if not ok:
        want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
        raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")


def _rows_at_least(t: torch.Tensor, rows: int, name: str):
    if t.dim() != 2 or t.shape[0] < rows:
        raise ValueError(f"{name} must be 2-D with at least {rows} rows, got {list(t.shape)}")


def _i32_host(a) -> ctypes.c_void_p:
    import numpy as np
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def check_decode_tables(ctx_lens, block_table, num_pages: int, max_ctx_len: int) -> int:
    """rlq_check_decode_tables on host arrays; returns the RLQ_* status."""
    cl, pc = _i32_host(ctx_lens)
    bt, pb = _i32_host(block_table)
    return lib().rlq_check_decode_tables(len(cl), pc, pb, bt.shape[1], num_pages, max_ctx_len)


def check_append_tables(cu_seqlens, start_pos, block_table, num_pages: int, n_tokens: int) -> int:
    """rlq_check_append_tables on host arrays; returns the RLQ_* status."""
    cu, pc = _i32_host(cu_seqlens)
    sp, ps = _i32_host(start_pos)
    bt, pb = _i32_host(block_table)
    if len(cu) != len(sp) + 1:
        return RLQ_EINVAL
    return lib().rlq_check_append_tables(len(sp), pc, ps, pb, bt.shape[1], num_pages, n_tokens)


def check_extend_tables(cu_seqlens_q, ctx_lens, block_table, num_pages: int, max_q_len: int,
                        max_ctx_len: int) -> int:
    """rlq_check_extend_tables on host arrays; returns the RLQ_* status."""
    cq, pq = _i32_host(cu_seqlens_q)
    cl, pc = _i32_host(ctx_lens)
    bt, pb = _i32_host(block_table)
    if len(cq) != len(cl) + 1:
        return RLQ_EINVAL
    return lib().rlq_check_extend_tables(len(cl), pq, pc, pb, bt.shape[1], num_pages, max_q_len, max_ctx_len)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def abi_version() -> int:
    return lib().rlq_abi_version()


def default_params() -> LayerParams:
    return lib().rlq_layer_params_default()


def params(tau: float, gain: float, level_inner: float = 0.4528, level_outer: float = 1.510) -> LayerParams:
    return LayerParams(tau, gain, level_inner, level_outer)


def coupled_gain(tau: float, level_inner: float = 0.4528, level_outer: float = 1.510) -> float:
    return lib().rlq_coupled_gain(tau, level_inner, level_outer)


@dataclass
class PagedCache:
    """Device pools of one layer (layouts of include/rlq.h)."""
    codes: torch.Tensor                 # int32 [P][64][32] (uint32 bit patterns)
    meta: torch.Tensor                  # float32 [P][64][8]
    rope: torch.Tensor                  # bfloat16 [P][64][64]
    sink: torch.Tensor | None = None    # bfloat16 [max_batch][n_sink][512]
    recent: torch.Tensor | None = None  # bfloat16 [max_batch][n_recent][512]

    @classmethod
    def allocate(cls, num_pages: int, *, max_batch: int = 0, n_sink: int = 0, n_recent: int = 0,
                 device="cuda", zero: bool = True) -> "PagedCache":
        mk = torch.zeros if zero else torch.empty
        return cls(
            codes=mk((num_pages, PAGE, WORDS), dtype=torch.int32, device=device),
            meta=mk((num_pages, PAGE, 2 * NGROUPS), dtype=torch.float32, device=device),
            rope=mk((num_pages, PAGE, DR), dtype=torch.bfloat16, device=device),
            sink=mk((max_batch, n_sink, DC), dtype=torch.bfloat16, device=device) if n_sink else None,
            recent=mk((max_batch, n_recent, DC), dtype=torch.bfloat16, device=device) if n_recent else None)

    @property
    def num_pages(self) -> int:
        return self.codes.shape[0]

    def desc(self) -> CacheDesc:
        _shape(self.codes, (None, PAGE, WORDS), "codes")
        _shape(self.meta, (self.num_pages, PAGE, 2 * NGROUPS), "meta")
        _shape(self.rope, (self.num_pages, PAGE, DR), "rope")
        _shape(self.sink, (None, None, DC), "sink")
        _shape(self.recent, (None, None, DC), "recent")
        if self.sink is not None and self.recent is not None and self.sink.shape[0] != self.recent.shape[0]:
            raise ValueError("sink and recent must have the same max_batch")
        mb = 0
        for t in (self.sink, self.recent):
            if t is not None:
                mb = t.shape[0]
        return CacheDesc(
            _ptr(self.codes, torch.int32, "codes"), _ptr(self.meta, torch.float32, "meta"),
            _ptr(self.rope, torch.bfloat16, "rope"), self.num_pages, self.codes.shape[1],
            _ptr(self.sink, torch.bfloat16, "sink"), _ptr(self.recent, torch.bfloat16, "recent"),
            0 if self.sink is None else self.sink.shape[1],
            0 if self.recent is None else self.recent.shape[1], mb)


def quantize_append(p: LayerParams, cache: PagedCache, k_rope: torch.Tensor,
                    cu_seqlens: torch.Tensor, start_pos: torch.Tensor, block_table: torch.Tensor,
                    *, latent: torch.Tensor | None = None, latent_rot: torch.Tensor | None = None,
                    rotation: torch.Tensor | None = None, n_tokens: int | None = None,
                    z_debug: torch.Tensor | None = None, stream=None) -> None:
    """rlq_quantize_append (see include/rlq.h)."""
    if n_tokens is None:
        n_tokens = k_rope.shape[0]
    n, batch = int(n_tokens), start_pos.shape[0] if start_pos.dim() == 1 else -1
    _shape(start_pos, (None,), "start_pos")
    _shape(cu_seqlens, (batch + 1,), "cu_seqlens")
    _rows_at_least(block_table, batch, "block_table")
    # Token arrays hold at least n_tokens rows (the call reads the first n_tokens).
    for t, w, name in ((k_rope, DR, "k_rope"), (latent, DC, "latent"), (latent_rot, DC, "latent_rot"),
                       (z_debug, DC, "z_debug")):
        if t is not None:
            _shape(t, (None, w), name)
            _rows_at_least(t, n, name)
    _shape(rotation, (DC, DC), "rotation")
    desc = cache.desc()
    st = lib().rlq_quantize_append(
        ctypes.byref(p), ctypes.byref(desc), _ptr(latent, torch.bfloat16, "latent"),
        _ptr(latent_rot, torch.float32, "latent_rot"), _ptr(rotation, torch.bfloat16, "rotation"),
        _ptr(k_rope, torch.bfloat16, "k_rope"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        _ptr(start_pos, torch.int32, "start_pos"), _ptr(block_table, torch.int32, "block_table"),
        block_table.shape[1], start_pos.shape[0], int(n_tokens),
        _ptr(z_debug, torch.float32, "z_debug"), _stream(stream))
    _check(st, "rlq_quantize_append")


def decode_workspace_size(batch: int, heads: int, max_ctx_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rlq_mla_decode_workspace_size(batch, heads, max_ctx_len, ctypes.byref(n)),
           "rlq_mla_decode_workspace_size")
    return n.value


def _decode_shapes(q_c, q_r, block_table, ctx_lens, out, lse):
    """Shapes of a decode call's tensors; returns (batch, heads)."""
    if q_c.dim() != 3:
        raise ValueError(f"q_c must have shape [batch, heads, {DC}], got {list(q_c.shape)}")
    batch, heads = int(q_c.shape[0]), int(q_c.shape[1])
    _shape(q_c, (batch, heads, DC), "q_c")
    _shape(q_r, (batch, heads, DR), "q_r")
    _shape(ctx_lens, (batch,), "ctx_lens")
    _rows_at_least(block_table, batch, "block_table")
    _shape(out, (batch, heads, DC), "out")
    _shape(lse, (batch, heads), "lse")
    return batch, heads


def mla_decode(p: LayerParams, cache: PagedCache, q_c: torch.Tensor, q_r: torch.Tensor,
               sm_scale: float, block_table: torch.Tensor, ctx_lens: torch.Tensor,
               max_ctx_len: int, *, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
               want_lse: bool = True, workspace: torch.Tensor | None = None, stream=None):
    """rlq_mla_decode (see include/rlq.h).  Returns (out, lse)."""
    batch, heads = _decode_shapes(q_c, q_r, block_table, ctx_lens, out, lse)
    if out is None:
        out = torch.empty((batch, heads, DC), dtype=torch.float32, device=q_c.device)
    if lse is None and want_lse:
        lse = torch.empty((batch, heads), dtype=torch.float32, device=q_c.device)
    need = decode_workspace_size(batch, heads, max_ctx_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_c.device)
    desc = cache.desc()
    st = lib().rlq_mla_decode(
        ctypes.byref(p), ctypes.byref(desc), _ptr(q_c, torch.bfloat16, "q_c"),
        _ptr(q_r, torch.bfloat16, "q_r"), batch, heads, float(sm_scale),
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), int(max_ctx_len),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "rlq_mla_decode")
    return out, lse


def mla_decode_noalloc(p: LayerParams, cache: PagedCache, q_c: torch.Tensor, q_r: torch.Tensor,
                       sm_scale: float, block_table: torch.Tensor, ctx_lens: torch.Tensor,
                       max_ctx_len: int, *, out: torch.Tensor, lse: torch.Tensor | None = None, stream=None):
    """rlq_mla_decode_noalloc (see include/rlq.h): rlq_mla_decode with the
    library's static scratch instead of a workspace; `out` (and `lse`) are
    caller-allocated, so the call allocates nothing.  Returns (out, lse)."""
    batch, heads = _decode_shapes(q_c, q_r, block_table, ctx_lens, out, lse)
    desc = cache.desc()
    st = lib().rlq_mla_decode_noalloc(
        ctypes.byref(p), ctypes.byref(desc), _ptr(q_c, torch.bfloat16, "q_c"),
        _ptr(q_r, torch.bfloat16, "q_r"), batch, heads, float(sm_scale),
        _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), int(max_ctx_len),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream))
    if st == RLQ_ENOSPC:
        need = decode_workspace_size(batch, heads, max_ctx_len)
        raise RlqError(st, f"rlq_mla_decode_noalloc (needs {need} bytes of scratch, "
                           f"the static array holds {NOALLOC_SCRATCH_BYTES})")
    _check(st, "rlq_mla_decode_noalloc")
    return out, lse


def extend_workspace_size(batch: int, heads: int, max_q_len: int, max_ctx_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().rlq_mla_extend_workspace_size(batch, heads, max_q_len, max_ctx_len, ctypes.byref(n)),
           "rlq_mla_extend_workspace_size")
    return n.value


def mla_extend(p: LayerParams, cache: PagedCache, q_c: torch.Tensor, q_r: torch.Tensor,
               cu_seqlens_q: torch.Tensor, max_q_len: int, sm_scale: float, block_table: torch.Tensor,
               ctx_lens: torch.Tensor, max_ctx_len: int, *, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, want_lse: bool = True,
               workspace: torch.Tensor | None = None, stream=None):
    """rlq_mla_extend (see include/rlq.h): q_c [total_q][heads][512].  Returns (out, lse)."""
    if q_c.dim() != 3 or cu_seqlens_q.dim() != 1:
        raise ValueError("q_c must be [total_q, heads, 512] and cu_seqlens_q 1-D")
    total_q, heads = int(q_c.shape[0]), int(q_c.shape[1])
    batch = cu_seqlens_q.shape[0] - 1
    _shape(q_c, (total_q, heads, DC), "q_c")
    _shape(q_r, (total_q, heads, DR), "q_r")
    _shape(ctx_lens, (batch,), "ctx_lens")
    _rows_at_least(block_table, batch, "block_table")
    _shape(out, (total_q, heads, DC), "out")
    _shape(lse, (total_q, heads), "lse")
    if out is None:
        out = torch.empty((total_q, heads, DC), dtype=torch.float32, device=q_c.device)
    if lse is None and want_lse:
        lse = torch.empty((total_q, heads), dtype=torch.float32, device=q_c.device)
    need = extend_workspace_size(batch, heads, max_q_len, max_ctx_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_c.device)
    desc = cache.desc()
    st = lib().rlq_mla_extend(
        ctypes.byref(p), ctypes.byref(desc), _ptr(q_c, torch.bfloat16, "q_c"),
        _ptr(q_r, torch.bfloat16, "q_r"), _ptr(cu_seqlens_q, torch.int32, "cu_seqlens_q"), batch, heads,
        int(max_q_len), float(sm_scale), _ptr(block_table, torch.int32, "block_table"), block_table.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), int(max_ctx_len),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "rlq_mla_extend")
    return out, lse
