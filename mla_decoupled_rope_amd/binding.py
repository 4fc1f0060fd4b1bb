"""Thin ctypes binding over libmla.so (the C ABI in include/mla.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current HIP
stream.  If the library is missing, importing this module raises: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("work_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("position_scale", ctypes.c_float), ("rope_base", ctypes.c_double),
    ]


class PagedCache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_decoupled_rope_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    pd, pc = ctypes.POINTER(Dims), ctypes.POINTER(PagedCache)
    sig = {
        "mla_rope_apply": [pd, pc, vp, vp, i64, vp, vp, vp, vp, vp, i64, vp],
        "mla_absorb_q": [pd, vp, vp, i64, vp, vp],
        "mla_rope_absorb_q": [pd, pc, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, i64, vp],
        "mla_decode": [pd, pc, vp, vp, vp, i32, vp, vp, vp, sz, vp],
        "mla_decode_noalloc": [pd, pc, vp, vp, vp, i32, vp, vp, vp],
        "mla_decode_proj": [pd, pc, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "mla_decode_split_kv": [pd, pc, vp, vp, vp, i32, vp, sz, vp],
        "mla_merge_out_proj": [pd, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "mla_prefill": [pd, pc, vp, vp, vp, vp, vp, i32, vp, vp, vp],
        "mla_out_proj": [pd, vp, vp, i64, vp, vp],
        "mla_decode_plan": [pd, i32, vp, ctypes.POINTER(i32), ctypes.POINTER(i64)],
        "mla_prefill_mha": [pd, pc, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp],
        "mla_kv_project": [pd, pc, vp, i64, i32, vp, vp, vp, vp, vp, sz, vp],
        "mla_q_project": [pd, vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "mla_q_project_folded": [pd, vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        "mla_fold_q_weights": [pd, i32, vp, vp, vp, vp],
        "mla_cache_write_per_head": [pd, pc, vp, vp, vp, vp, i64, vp],
        "mla_decode_per_head": [pd, pc, vp, vp, vp, i32, vp, vp, vp, sz, vp],
        "mla_decode_per_head_proj": [pd, pc, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [pd, i32, vp]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode_proj_workspace_size.argtypes = [pd, i32, vp]
    lib.mla_decode_proj_workspace_size.restype = sz
    lib.mla_prefill_mha_workspace_size.argtypes = [pd, i32, vp, vp]
    lib.mla_prefill_mha_workspace_size.restype = sz
    lib.mla_front_workspace_size.argtypes = [pd, i64, i32, i32]
    lib.mla_front_workspace_size.restype = sz
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()

EXPORTS = ("mla_rope_apply", "mla_absorb_q", "mla_rope_absorb_q", "mla_decode_workspace_size", "mla_decode", "mla_decode_noalloc",
           "mla_decode_proj_workspace_size", "mla_decode_proj", "mla_decode_split_kv", "mla_merge_out_proj",
           "mla_prefill",
           "mla_out_proj", "mla_status_string", "mla_last_error", "mla_decode_plan",
           "mla_prefill_mha_workspace_size", "mla_prefill_mha", "mla_front_workspace_size", "mla_kv_project",
           "mla_q_project", "mla_q_project_folded", "mla_fold_q_weights", "mla_cache_write_per_head",
           "mla_decode_per_head", "mla_decode_per_head_proj")


def _check(status: int):
    if status != 0:
        raise MLAError(status, LIB.mla_last_error().decode())


@dataclass(frozen=True)
class MLADims:
    """Python mirror of mla_dims."""

    n_heads: int
    d_head: int
    d_v: int
    d_latent: int
    d_rope: int
    dtype: torch.dtype = torch.bfloat16
    softmax_scale: float | None = None
    position_scale: float | None = None  # None: softmax_scale (one scale on the summed score)
    rope_base: float = 10000.0
    page_size: int = 64
    # dtype of q_lat (None: same as dtype).  torch.float32 with a bf16 dtype is
    # the float32 working precision (two-term q~ and softmax weights).
    work_dtype: torch.dtype | None = None

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def wdtype(self) -> torch.dtype:
        return self.dtype if self.work_dtype is None else self.work_dtype

    def c(self) -> Dims:
        scale = self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.d_head + self.d_rope)
        code = {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16}
        return Dims(self.n_heads, self.d_head, self.d_v, self.d_latent, self.d_rope, self.page_size,
                    code[self.dtype], code[self.wdtype], scale,
                    scale if self.position_scale is None else self.position_scale, self.rope_base)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _host_i32(t: torch.Tensor, name: str):
    if t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous host int32 tensor")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _cache(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, row: int | None = None) -> PagedCache:
    row = dims.row if row is None else row
    _dev(cache, "cache", dims.dtype)
    if cache.dim() != 3 or cache.shape[1] != dims.page_size or cache.shape[2] != row:
        raise ValueError(f"cache must be [num_pages, {dims.page_size}, {row}]")
    _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_pages_per_seq]")
    return PagedCache(cache.data_ptr(), cache.shape[0], block_table.data_ptr(), block_table.shape[0],
                      block_table.shape[1])


def rope_apply(dims: MLADims, cache: torch.Tensor | None, block_table: torch.Tensor | None,
               q_rope: torch.Tensor | None = None, q_pos: torch.Tensor | None = None,
               q_lat: torch.Tensor | None = None, kv_latent: torch.Tensor | None = None,
               k_rope: torch.Tensor | None = None, kv_seq: torch.Tensor | None = None,
               kv_pos: torch.Tensor | None = None) -> None:
    """mla_rope_apply: rotate q^R into q_lat[..., d_c:] and write [c | R k^R] rows into the cache."""
    n_q = 0 if q_rope is None else q_rope.shape[0]
    n_kv = 0 if kv_latent is None else kv_latent.shape[0]
    if n_q:
        _dev(q_rope, "q_rope", dims.dtype, (n_q, dims.n_heads, dims.d_rope))
        _dev(q_pos, "q_pos", torch.int32, (n_q,))
        _dev(q_lat, "q_lat", dims.wdtype, (n_q, dims.n_heads, dims.row))
    cstruct = None
    if n_kv:
        cstruct = _cache(dims, cache, block_table)
        _dev(kv_latent, "kv_latent", dims.dtype, (n_kv, dims.d_latent))
        _dev(k_rope, "k_rope", dims.dtype, (n_kv, dims.d_rope))
        _dev(kv_seq, "kv_seq", torch.int32, (n_kv,))
        _dev(kv_pos, "kv_pos", torch.int32, (n_kv,))
    d = dims.c()
    _check(LIB.mla_rope_apply(ctypes.byref(d), ctypes.byref(cstruct) if cstruct else None,
                              _ptr(q_rope) if n_q else None, _ptr(q_pos) if n_q else None, n_q,
                              _ptr(q_lat) if n_q else None, _ptr(kv_latent) if n_kv else None,
                              _ptr(k_rope) if n_kv else None, _ptr(kv_seq) if n_kv else None,
                              _ptr(kv_pos) if n_kv else None, n_kv, _stream()))


def absorb_q(dims: MLADims, q_nope: torch.Tensor, w_uk: torch.Tensor, q_lat: torch.Tensor) -> None:
    """mla_absorb_q: q_lat[n, h, :d_c] = W_UK[h]^T q_nope[n, h]."""
    n = q_nope.shape[0]
    _dev(q_nope, "q_nope", dims.dtype, (n, dims.n_heads, dims.d_head))
    _dev(w_uk, "w_uk", dims.dtype, (dims.n_heads, dims.d_head, dims.d_latent))
    _dev(q_lat, "q_lat", dims.wdtype, (n, dims.n_heads, dims.row))
    d = dims.c()
    _check(LIB.mla_absorb_q(ctypes.byref(d), q_nope.data_ptr(), w_uk.data_ptr(), n, q_lat.data_ptr(), _stream()))


def rope_absorb_q(dims: MLADims, cache: torch.Tensor | None, block_table: torch.Tensor | None,
                  q_nope: torch.Tensor, w_uk: torch.Tensor, q_rope: torch.Tensor, q_pos: torch.Tensor,
                  q_lat: torch.Tensor, kv_latent: torch.Tensor | None = None, k_rope: torch.Tensor | None = None,
                  kv_seq: torch.Tensor | None = None, kv_pos: torch.Tensor | None = None) -> None:
    """mla_rope_absorb_q: rope_apply and absorb_q in one launch (bit-identical results)."""
    n_q = q_nope.shape[0]
    n_kv = 0 if kv_latent is None else kv_latent.shape[0]
    _dev(q_nope, "q_nope", dims.dtype, (n_q, dims.n_heads, dims.d_head))
    _dev(w_uk, "w_uk", dims.dtype, (dims.n_heads, dims.d_head, dims.d_latent))
    _dev(q_rope, "q_rope", dims.dtype, (n_q, dims.n_heads, dims.d_rope))
    _dev(q_pos, "q_pos", torch.int32, (n_q,))
    _dev(q_lat, "q_lat", dims.wdtype, (n_q, dims.n_heads, dims.row))
    cstruct = None
    if n_kv:
        cstruct = _cache(dims, cache, block_table)
        _dev(kv_latent, "kv_latent", dims.dtype, (n_kv, dims.d_latent))
        _dev(k_rope, "k_rope", dims.dtype, (n_kv, dims.d_rope))
        _dev(kv_seq, "kv_seq", torch.int32, (n_kv,))
        _dev(kv_pos, "kv_pos", torch.int32, (n_kv,))
    d = dims.c()
    _check(LIB.mla_rope_absorb_q(ctypes.byref(d), ctypes.byref(cstruct) if cstruct else None, _ptr(q_nope),
                                 _ptr(w_uk), _ptr(q_rope), _ptr(q_pos), n_q, _ptr(q_lat),
                                 _ptr(kv_latent) if n_kv else None, _ptr(k_rope) if n_kv else None,
                                 _ptr(kv_seq) if n_kv else None, _ptr(kv_pos) if n_kv else None, n_kv, _stream()))


def decode_plan(dims: MLADims, seq_lens_host: torch.Tensor):
    _host_i32(seq_lens_host, "seq_lens_host")
    d = dims.c()
    sp, ni = ctypes.c_int32(), ctypes.c_int64()
    _check(LIB.mla_decode_plan(ctypes.byref(d), seq_lens_host.numel(), seq_lens_host.data_ptr(),
                               ctypes.byref(sp), ctypes.byref(ni)))
    return sp.value, ni.value


def decode_workspace_size(dims: MLADims, seq_lens_host: torch.Tensor) -> int:
    _host_i32(seq_lens_host, "seq_lens_host")
    d = dims.c()
    return int(LIB.mla_decode_workspace_size(ctypes.byref(d), seq_lens_host.numel(), seq_lens_host.data_ptr()))


def decode_workspace(dims: MLADims, seq_lens_host: torch.Tensor, device="cuda") -> torch.Tensor | None:
    n = decode_workspace_size(dims, seq_lens_host)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def decode_proj_workspace_size(dims: MLADims, seq_lens_host: torch.Tensor) -> int:
    _host_i32(seq_lens_host, "seq_lens_host")
    d = dims.c()
    return int(LIB.mla_decode_proj_workspace_size(ctypes.byref(d), seq_lens_host.numel(), seq_lens_host.data_ptr()))


def decode_proj_workspace(dims: MLADims, seq_lens_host: torch.Tensor, device="cuda") -> torch.Tensor | None:
    n = decode_proj_workspace_size(dims, seq_lens_host)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def decode_proj(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
                seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> None:
    """mla_decode_proj: out[b, h] = W_UV[h] (sum_t softmax(s)_t c_t), the split merge and the
    output absorption in one launch (obar is not written)."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(w_uv, "w_uv", dims.dtype, (dims.n_heads, dims.d_v, dims.d_latent))
    _dev(out, "out", torch.float32, (batch, dims.n_heads, dims.d_v))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_decode_proj(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                               seq_lens_host.data_ptr(), batch, w_uv.data_ptr(), out.data_ptr(), _ptr(lse),
                               _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))


def decode_split_kv(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
                    seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, workspace: torch.Tensor | None) -> None:
    """mla_decode_split_kv: mla_decode_proj's split attention alone; every work item's partial
    goes to the workspace (mla_decode_proj_workspace_size bytes) for merge_out_proj."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_decode_split_kv(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                                   seq_lens_host.data_ptr(), batch, _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream()))


def merge_out_proj(dims: MLADims, seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, w_uv: torch.Tensor,
                   out: torch.Tensor, lse: torch.Tensor | None, workspace: torch.Tensor | None) -> None:
    """mla_merge_out_proj: mla_decode_proj's split merge and output absorption alone, from the
    workspace decode_split_kv filled."""
    batch = seq_lens_host.numel()
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(w_uv, "w_uv", dims.dtype, (dims.n_heads, dims.d_v, dims.d_latent))
    _dev(out, "out", torch.float32, (batch, dims.n_heads, dims.d_v))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_merge_out_proj(ctypes.byref(d), seq_lens.data_ptr(), seq_lens_host.data_ptr(), batch,
                                  w_uv.data_ptr(), out.data_ptr(), _ptr(lse), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream()))


def decode(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
           seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, out_latent: torch.Tensor,
           lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> None:
    """mla_decode: out_latent[b] = sum_t softmax(s)_t c_t over positions 0 .. seq_lens[b]-1."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(out_latent, "out_latent", torch.float32, (batch, dims.n_heads, dims.d_latent))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_decode(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                          seq_lens_host.data_ptr(), batch, out_latent.data_ptr(), _ptr(lse), _ptr(workspace),
                          0 if workspace is None else workspace.numel(), _stream()))


def decode_noalloc(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
                   seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, out_latent: torch.Tensor,
                   lse: torch.Tensor | None = None) -> None:
    """mla_decode_noalloc: mla_decode with the split partials in the library's fixed device scratch."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(out_latent, "out_latent", torch.float32, (batch, dims.n_heads, dims.d_latent))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    d = dims.c()
    _check(LIB.mla_decode_noalloc(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                                  seq_lens_host.data_ptr(), batch, out_latent.data_ptr(), _ptr(lse), _stream()))


def per_head_row(dims: MLADims) -> int:
    """Elements per cache row with one position key per head: d_latent + n_heads * d_rope."""
    return dims.d_latent + dims.n_heads * dims.d_rope


def cache_write_per_head(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, kv_latent: torch.Tensor,
                         k_rope: torch.Tensor, kv_seq: torch.Tensor, kv_pos: torch.Tensor) -> None:
    """mla_cache_write_per_head: rows [c | R_t k^R_{t,0} | ... | R_t k^R_{t,H-1}] into a per-head-key cache."""
    n = kv_latent.shape[0]
    cstruct = _cache(dims, cache, block_table, per_head_row(dims))
    _dev(kv_latent, "kv_latent", dims.dtype, (n, dims.d_latent))
    _dev(k_rope, "k_rope", dims.dtype, (n, dims.n_heads, dims.d_rope))
    _dev(kv_seq, "kv_seq", torch.int32, (n,))
    _dev(kv_pos, "kv_pos", torch.int32, (n,))
    d = dims.c()
    _check(LIB.mla_cache_write_per_head(ctypes.byref(d), ctypes.byref(cstruct), kv_latent.data_ptr(),
                                        k_rope.data_ptr(), kv_seq.data_ptr(), kv_pos.data_ptr(), n, _stream()))


def decode_per_head(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
                    seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, out_latent: torch.Tensor,
                    lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> None:
    """mla_decode_per_head: decode over a cache with one position key per head."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table, per_head_row(dims))
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(out_latent, "out_latent", torch.float32, (batch, dims.n_heads, dims.d_latent))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_decode_per_head(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                                   seq_lens_host.data_ptr(), batch, out_latent.data_ptr(), _ptr(lse),
                                   _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))


def decode_per_head_proj(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
                         seq_lens: torch.Tensor, seq_lens_host: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor,
                         lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> None:
    """mla_decode_per_head_proj: decode over per-head position keys, then the split merge
    and the output absorption in one launch (workspace of decode_proj_workspace_size)."""
    batch = seq_lens_host.numel()
    cstruct = _cache(dims, cache, block_table, per_head_row(dims))
    _dev(q_lat, "q_lat", dims.wdtype, (batch, dims.n_heads, dims.row))
    _dev(seq_lens, "seq_lens", torch.int32, (batch,))
    _host_i32(seq_lens_host, "seq_lens_host")
    _dev(w_uv, "w_uv", dims.dtype, (dims.n_heads, dims.d_v, dims.d_latent))
    _dev(out, "out", torch.float32, (batch, dims.n_heads, dims.d_v))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_decode_per_head_proj(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), seq_lens.data_ptr(),
                                        seq_lens_host.data_ptr(), batch, w_uv.data_ptr(), out.data_ptr(), _ptr(lse),
                                        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))


def prefill(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_lat: torch.Tensor,
            cu_q: torch.Tensor, q_start: torch.Tensor, cu_q_host: torch.Tensor, q_start_host: torch.Tensor,
            out_latent: torch.Tensor, lse: torch.Tensor | None = None) -> None:
    """mla_prefill: causal absorbed attention for new query chunks over the cache."""
    batch = q_start_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _host_i32(cu_q_host, "cu_q_host")
    _host_i32(q_start_host, "q_start_host")
    if cu_q_host.numel() != batch + 1:
        raise ValueError("cu_q must have batch + 1 entries")
    n = int(cu_q_host[-1])
    _dev(q_lat, "q_lat", dims.wdtype, (n, dims.n_heads, dims.row))
    _dev(cu_q, "cu_q", torch.int32, (batch + 1,))
    _dev(q_start, "q_start", torch.int32, (batch,))
    _dev(out_latent, "out_latent", torch.float32, (n, dims.n_heads, dims.d_latent))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (n, dims.n_heads))
    d = dims.c()
    _check(LIB.mla_prefill(ctypes.byref(d), ctypes.byref(cstruct), q_lat.data_ptr(), cu_q.data_ptr(),
                           q_start.data_ptr(), cu_q_host.data_ptr(), q_start_host.data_ptr(), batch,
                           out_latent.data_ptr(), _ptr(lse), _stream()))


def prefill_mha_workspace_size(dims: MLADims, cu_q_host: torch.Tensor, q_start_host: torch.Tensor) -> int:
    _host_i32(cu_q_host, "cu_q_host")
    _host_i32(q_start_host, "q_start_host")
    d = dims.c()
    n = int(LIB.mla_prefill_mha_workspace_size(ctypes.byref(d), q_start_host.numel(), cu_q_host.data_ptr(),
                                               q_start_host.data_ptr()))
    if n == 0 and int(cu_q_host[-1]) + int(q_start_host.sum()) > 0:
        raise MLAError(2, LIB.mla_last_error().decode())
    return n


def prefill_mha_workspace(dims: MLADims, cu_q_host: torch.Tensor, q_start_host: torch.Tensor,
                          device="cuda") -> torch.Tensor | None:
    n = prefill_mha_workspace_size(dims, cu_q_host, q_start_host)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def prefill_mha(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, q_nope: torch.Tensor,
                q_lat: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor, cu_q: torch.Tensor,
                q_start: torch.Tensor, cu_q_host: torch.Tensor, q_start_host: torch.Tensor, out: torch.Tensor,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> None:
    """mla_prefill_mha: causal prefill in the materialised form; out[n, h] = sum_t alpha_t W_UV[h] c_t (float32)."""
    batch = q_start_host.numel()
    cstruct = _cache(dims, cache, block_table)
    _host_i32(cu_q_host, "cu_q_host")
    _host_i32(q_start_host, "q_start_host")
    if cu_q_host.numel() != batch + 1:
        raise ValueError("cu_q must have batch + 1 entries")
    n = int(cu_q_host[-1])
    _dev(q_nope, "q_nope", dims.dtype, (n, dims.n_heads, dims.d_head))
    _dev(q_lat, "q_lat", dims.wdtype, (n, dims.n_heads, dims.row))
    _dev(w_uk, "w_uk", dims.dtype, (dims.n_heads, dims.d_head, dims.d_latent))
    _dev(w_uv, "w_uv", dims.dtype, (dims.n_heads, dims.d_v, dims.d_latent))
    _dev(cu_q, "cu_q", torch.int32, (batch + 1,))
    _dev(q_start, "q_start", torch.int32, (batch,))
    _dev(out, "out", torch.float32, (n, dims.n_heads, dims.d_v))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (n, dims.n_heads))
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_prefill_mha(ctypes.byref(d), ctypes.byref(cstruct), q_nope.data_ptr(), q_lat.data_ptr(),
                               w_uk.data_ptr(), w_uv.data_ptr(), cu_q.data_ptr(), q_start.data_ptr(),
                               cu_q_host.data_ptr(), q_start_host.data_ptr(), batch, out.data_ptr(), _ptr(lse),
                               _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))


def out_proj(dims: MLADims, out_latent: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor) -> None:
    """mla_out_proj: out[n, h] = W_UV[h] out_latent[n, h] (out_latent and out are float32)."""
    n = out_latent.shape[0]
    _dev(out_latent, "out_latent", torch.float32, (n, dims.n_heads, dims.d_latent))
    _dev(w_uv, "w_uv", dims.dtype, (dims.n_heads, dims.d_v, dims.d_latent))
    _dev(out, "out", torch.float32, (n, dims.n_heads, dims.d_v))
    d = dims.c()
    _check(LIB.mla_out_proj(ctypes.byref(d), out_latent.data_ptr(), w_uv.data_ptr(), n, out.data_ptr(), _stream()))


def front_workspace_size(dims: MLADims, n: int, d_model: int, d_qlat: int = 0) -> int:
    d = dims.c()
    size = int(LIB.mla_front_workspace_size(ctypes.byref(d), n, d_model, d_qlat))
    if size == 0 and n > 0:
        raise MLAError(2, LIB.mla_last_error().decode())
    return size


def front_workspace(dims: MLADims, n: int, d_model: int, d_qlat: int = 0, device="cuda") -> torch.Tensor:
    return torch.empty(max(front_workspace_size(dims, n, d_model, d_qlat), 1), dtype=torch.uint8, device=device)


def kv_project(dims: MLADims, cache: torch.Tensor, block_table: torch.Tensor, h: torch.Tensor, w_dkv: torch.Tensor,
               w_kr: torch.Tensor, kv_seq: torch.Tensor, kv_pos: torch.Tensor, workspace: torch.Tensor) -> None:
    """mla_kv_project: cache row of (kv_seq[j], kv_pos[j]) = [W_DKV h[j] | R_pos W_KR h[j]]."""
    n, d_model = h.shape
    cstruct = _cache(dims, cache, block_table)
    _dev(h, "h", dims.dtype, (n, d_model))
    _dev(w_dkv, "w_dkv", dims.dtype, (dims.d_latent, d_model))
    _dev(w_kr, "w_kr", dims.dtype, (dims.d_rope, d_model))
    _dev(kv_seq, "kv_seq", torch.int32, (n,))
    _dev(kv_pos, "kv_pos", torch.int32, (n,))
    _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_kv_project(ctypes.byref(d), ctypes.byref(cstruct), h.data_ptr(), n, d_model, w_dkv.data_ptr(),
                              w_kr.data_ptr(), kv_seq.data_ptr(), kv_pos.data_ptr(), workspace.data_ptr(),
                              workspace.numel(), _stream()))


def q_project(dims: MLADims, h: torch.Tensor, w_dq: torch.Tensor, w_uq: torch.Tensor, w_qr: torch.Tensor,
              q_pos: torch.Tensor, q_nope: torch.Tensor, q_lat: torch.Tensor, workspace: torch.Tensor) -> None:
    """mla_q_project: q_nope = W_UQ (W_DQ h), q_lat tail = R_pos W_QR (W_DQ h)."""
    n, d_model = h.shape
    d_qlat = w_dq.shape[0]
    _dev(h, "h", dims.dtype, (n, d_model))
    _dev(w_dq, "w_dq", dims.dtype, (d_qlat, d_model))
    _dev(w_uq, "w_uq", dims.dtype, (dims.n_heads, dims.d_head, d_qlat))
    _dev(w_qr, "w_qr", dims.dtype, (dims.n_heads, dims.d_rope, d_qlat))
    _dev(q_pos, "q_pos", torch.int32, (n,))
    _dev(q_nope, "q_nope", dims.dtype, (n, dims.n_heads, dims.d_head))
    _dev(q_lat, "q_lat", dims.wdtype, (n, dims.n_heads, dims.row))
    _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_q_project(ctypes.byref(d), h.data_ptr(), n, d_model, d_qlat, w_dq.data_ptr(), w_uq.data_ptr(),
                             w_qr.data_ptr(), q_pos.data_ptr(), q_nope.data_ptr(), q_lat.data_ptr(),
                             workspace.data_ptr(), workspace.numel(), _stream()))


def q_project_folded(dims: MLADims, h: torch.Tensor, w_dq: torch.Tensor, w_fold: torch.Tensor, w_qr: torch.Tensor,
                     q_pos: torch.Tensor, q_lat: torch.Tensor, workspace: torch.Tensor) -> None:
    """mla_q_project_folded: q_lat = [W_fold (W_DQ h) | R_pos W_QR (W_DQ h)]."""
    n, d_model = h.shape
    d_qlat = w_dq.shape[0]
    _dev(h, "h", dims.dtype, (n, d_model))
    _dev(w_dq, "w_dq", dims.dtype, (d_qlat, d_model))
    _dev(w_fold, "w_fold", dims.dtype, (dims.n_heads, dims.d_latent, d_qlat))
    _dev(w_qr, "w_qr", dims.dtype, (dims.n_heads, dims.d_rope, d_qlat))
    _dev(q_pos, "q_pos", torch.int32, (n,))
    _dev(q_lat, "q_lat", dims.wdtype, (n, dims.n_heads, dims.row))
    _dev(workspace, "workspace", torch.uint8)
    d = dims.c()
    _check(LIB.mla_q_project_folded(ctypes.byref(d), h.data_ptr(), n, d_model, d_qlat, w_dq.data_ptr(),
                                    w_fold.data_ptr(), w_qr.data_ptr(), q_pos.data_ptr(), q_lat.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(), _stream()))


def fold_q_weights(dims: MLADims, w_uq: torch.Tensor, w_uk: torch.Tensor, w_fold: torch.Tensor) -> None:
    """mla_fold_q_weights: w_fold[i] = W_UK[i]^T W_UQ[i]."""
    d_qlat = w_uq.shape[2]
    _dev(w_uq, "w_uq", dims.dtype, (dims.n_heads, dims.d_head, d_qlat))
    _dev(w_uk, "w_uk", dims.dtype, (dims.n_heads, dims.d_head, dims.d_latent))
    _dev(w_fold, "w_fold", dims.dtype, (dims.n_heads, dims.d_latent, d_qlat))
    d = dims.c()
    _check(LIB.mla_fold_q_weights(ctypes.byref(d), d_qlat, w_uq.data_ptr(), w_uk.data_ptr(), w_fold.data_ptr(),
                                  _stream()))
