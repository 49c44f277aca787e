"""ctypes binding of libsmla.so (C ABI in include/smla.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is missing this module raises at import; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmla.so")

SMLA_OK = 0
SMLA_EINVAL = -1
SMLA_EUNSUPPORTED = -2
SMLA_EWORKSPACE = -3
SMLA_EHIP = -4
MAX_HEADS = 128
MAX_SPLIT = 32
RECORD_BYTES = 656

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m sparse_mla_decode_fp8_amd.build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_lib.sparse_mla_supported.argtypes = [_i32, _i32, _i32]
_lib.sparse_mla_supported.restype = ctypes.c_int
_lib.sparse_mla_workspace_bytes.argtypes = [_i32, _i32, _i64]
_lib.sparse_mla_workspace_bytes.restype = _i64
_lib.sparse_mla_split_for.argtypes = [_i32, _i32, _i64, _i32]
_lib.sparse_mla_split_for.restype = _i32
_lib.sparse_mla_fwd.argtypes = [
    _vp, _i64, _i64,        # q, strides
    _vp, _i64,              # kv, n_kv
    _vp, _vp, _i64,         # indptr, indices, nnz
    _i32, _i32, _f32, _i32,  # T, H, sm_scale, has_invalid
    _vp, _i64, _i64,        # out, strides
    _vp,                    # lse
    _vp, _i64,              # workspace, bytes
    _vp,                    # stream
]
_lib.sparse_mla_fwd.restype = ctypes.c_int
_lib.sparse_mla_fwd_noalloc.argtypes = [
    _vp, _i64, _i64,        # q, strides
    _vp, _i64,              # kv, n_kv
    _vp, _vp, _i64,         # indptr, indices, nnz
    _i32, _i32, _f32, _i32,  # T, H, sm_scale, has_invalid
    _vp, _i64, _i64,        # out, strides
    _vp,                    # lse
    _vp,                    # stream
]
_lib.sparse_mla_fwd_noalloc.restype = ctypes.c_int
NOALLOC_SCRATCH_BYTES = 64 << 20


class KvPool(ctypes.Structure):
    """smla_kv_pool: one paged pool of 656-byte records."""
    _fields_ = [("base", _vp), ("page_stride", _i64), ("page_records", _i64)]


_lib.sparse_mla_fwd_paged.argtypes = [
    _vp, _i64, _i64,        # q, strides
    ctypes.POINTER(KvPool),  # pools[2] (host)
    _vp, _vp, _i64,         # indptr, indices, nnz
    _i32, _i32, _f32, _i32,  # T, H, sm_scale, has_invalid
    _vp,                    # sink
    _vp, _i64, _i64,        # out, strides
    _vp,                    # lse
    _vp, _i64,              # workspace, bytes
    _vp,                    # stream
]
_lib.sparse_mla_fwd_paged.restype = ctypes.c_int
_lib.sparse_mla_v41_workspace_bytes.argtypes = [_i32, _i32, _i64]
_lib.sparse_mla_v41_workspace_bytes.restype = _i64
_lib.sparse_mla_fwd_v41.argtypes = [
    _vp, _i64, _i64,        # q, strides
    ctypes.POINTER(KvPool),  # pools[2] (host)
    _vp, _vp, _i64,         # indptr, indices, nnz
    _i32, _i32, _f32, _i32,  # T, H, sm_scale, has_invalid
    _vp, _vp, _vp, _i32,    # sink, pos, cos_sin, n_pos
    _vp, _vp, _vp, _vp,     # xo, xo_scales, lse, y_out
    _vp, _i64,              # workspace, bytes
    _vp,                    # stream
]
_lib.sparse_mla_fwd_v41.restype = ctypes.c_int
_lib.sparse_mla_mxfp8.argtypes = [_vp, _i64, _vp, _vp, _vp]
_lib.sparse_mla_mxfp8.restype = ctypes.c_int
_lib.sparse_mla_cache_write.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
_lib.sparse_mla_cache_write.restype = ctypes.c_int
_lib.sparse_mla_qk_probe.argtypes = [_vp, _vp, _i64, _vp, _i64, _i32, _vp, _vp]
_lib.sparse_mla_qk_probe.restype = ctypes.c_int
_lib.sparse_mla_decode_rows.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp]
_lib.sparse_mla_decode_rows.restype = ctypes.c_int
_lib.sparse_mla_last_error.argtypes = []
_lib.sparse_mla_last_error.restype = ctypes.c_char_p
_lib.sparse_mla_set_option.argtypes = [ctypes.c_char_p, _i64]
_lib.sparse_mla_set_option.restype = ctypes.c_int
_lib.sparse_mla_profile_begin.argtypes = [_i32]
_lib.sparse_mla_profile_begin.restype = ctypes.c_int
_lib.sparse_mla_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]
_lib.sparse_mla_profile_end.restype = ctypes.c_int

EXPORTED = (
    "sparse_mla_supported", "sparse_mla_workspace_bytes", "sparse_mla_split_for", "sparse_mla_fwd",
    "sparse_mla_fwd_noalloc",
    "sparse_mla_fwd_paged", "sparse_mla_v41_workspace_bytes", "sparse_mla_fwd_v41", "sparse_mla_mxfp8",
    "sparse_mla_cache_write", "sparse_mla_decode_rows", "sparse_mla_qk_probe", "sparse_mla_last_error", "sparse_mla_set_option",
    "sparse_mla_profile_begin", "sparse_mla_profile_end",
)


class SmlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"smla status {status}: {msg}")
        self.status = status


def _check(rc: int) -> None:
    if rc != SMLA_OK:
        raise SmlaError(rc, _lib.sparse_mla_last_error().decode(errors="replace"))


def lib() -> ctypes.CDLL:
    return _lib


def supported(num_heads: int, head_dim_qk: int = 576, dv: int = 512) -> bool:
    return bool(_lib.sparse_mla_supported(int(num_heads), int(head_dim_qk), int(dv)))


def workspace_bytes(T: int, H: int, nnz: int) -> int:
    n = _lib.sparse_mla_workspace_bytes(int(T), int(H), int(nnz))
    if n < 0:
        _check(int(n))
    return int(n)


def split_for(T: int, H: int, nnz: int, has_invalid: bool = False) -> int:
    """Chunks per row the forward uses for this shape on the current device."""
    n = _lib.sparse_mla_split_for(int(T), int(H), int(nnz), 1 if has_invalid else 0)
    if n < 0:
        _check(int(n))
    return int(n)


def set_option(name: str, value: int) -> None:
    _check(_lib.sparse_mla_set_option(name.encode(), int(value)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache = {}


def workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A device workspace of at least nbytes, reused per device and stream (the
    current stream of `device`, the one the call is queued on): calls on one
    stream are ordered, so they can share it, and calls on other streams get
    their own.  While the stream is being captured into a HIP graph the call
    gets a fresh workspace from the graph's own memory pool instead: graphs
    captured on one capture stream may be replayed on different streams at
    once, so they must not share a cached workspace."""
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    key = (device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def fwd(q: torch.Tensor, kv: torch.Tensor, indptr: torch.Tensor, indices: torch.Tensor,
        sm_scale: float, has_invalid: bool = False, return_lse: bool = True,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse MLA forward: q bf16 [T, H, 576], kv uint8 [N, 656], indptr int32 [T+1],
    indices int32 [nnz] -> (out bf16 [T, H, 512], lse f32 [T, H] or None)."""
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 576:
        raise ValueError("q must be bf16 [T, H, 576]")
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != RECORD_BYTES:
        raise ValueError(f"kv must be uint8 [N, {RECORD_BYTES}]")
    if not kv.is_contiguous():
        raise ValueError("kv rows must be contiguous")
    if indptr.dtype != torch.int32 or indices.dtype != torch.int32:
        raise ValueError("indptr and indices must be int32")
    if q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    dev = q.device
    for t in (kv, indptr, indices):
        if t.device != dev:
            raise ValueError("all tensors must be on q's device")
    T, H, _ = q.shape
    indptr = indptr.contiguous()
    indices = indices.contiguous()
    nnz = indices.numel()
    if indptr.numel() != T + 1:
        raise ValueError("indptr must have T + 1 entries")
    if out is None:
        out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    nbytes = workspace_bytes(T, H, nnz)
    if ws is None:
        ws = workspace(dev, nbytes)
    rc = _lib.sparse_mla_fwd(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(kv), kv.shape[0],
        _ptr(indptr), _ptr(indices) if nnz else None, nnz,
        T, H, float(sm_scale), 1 if has_invalid else 0,
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse),
        _ptr(ws), ws.numel(),
        _stream(dev))
    _check(rc)
    return out, lse


def fwd_noalloc(q: torch.Tensor, kv: torch.Tensor, indptr: torch.Tensor, indices: torch.Tensor,
                sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                has_invalid: bool = False) -> None:
    """sparse_mla_fwd_noalloc: the forward into the caller's out (bf16 [T, H, 512])
    and lse (f32 [T, H] or None), with the library's static per-device scratch
    in place of a workspace; nothing is allocated.  Calls that overlap on one
    device race on that scratch."""
    _check_fwd_args(q, indptr, indices)
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != RECORD_BYTES or not kv.is_contiguous():
        raise ValueError(f"kv must be contiguous uint8 [N, {RECORD_BYTES}]")
    T, H, _ = q.shape
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (T, H, 512) or out.stride(2) != 1:
        raise ValueError("out must be bf16 [T, H, 512] with a contiguous last dimension")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, H) or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous f32 [T, H]")
    for t in (kv, out) + ((lse,) if lse is not None else ()):
        if t.device != q.device:
            raise ValueError("all tensors must be on q's device")
    if not (indptr.is_contiguous() and indices.is_contiguous()):
        raise ValueError("indptr and indices must be contiguous (no copy is made)")
    nnz = indices.numel()
    rc = _lib.sparse_mla_fwd_noalloc(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(kv), kv.shape[0],
        _ptr(indptr), _ptr(indices) if nnz else None, nnz,
        T, H, float(sm_scale), 1 if has_invalid else 0,
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse),
        _stream(q.device))
    _check(rc)


def _check_fwd_args(q, indptr, indices):
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 576:
        raise ValueError("q must be bf16 [T, H, 576]")
    if indptr.dtype != torch.int32 or indices.dtype != torch.int32:
        raise ValueError("indptr and indices must be int32")
    if q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    for t in (indptr, indices):
        if t.device != q.device:
            raise ValueError("all tensors must be on q's device")
    if indptr.numel() != q.shape[0] + 1:
        raise ValueError("indptr must have T + 1 entries")


def fwd_paged(q: torch.Tensor, pools, indptr: torch.Tensor, indices: torch.Tensor,
              sm_scale: float, sink: Optional[torch.Tensor] = None, has_invalid: bool = False,
              return_lse: bool = True, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse MLA forward over two paged pools with an optional sink.

    pools: two (bytes, page_stride, page_records) triples, the window pool and
    the compressed pool; bytes is a contiguous uint8 device tensor holding the
    pool from page 0, or None for an absent pool.  Entries of indices: -1 no
    key, >= 0 a window-pool slot, other negative values a compressed-pool slot
    with bit 31 set.  sink: f32 [H] natural-log logits or None."""
    _check_fwd_args(q, indptr, indices)
    dev = q.device
    desc = _pool_descs(pools, dev)
    if sink is not None:
        if sink.dtype != torch.float32 or sink.numel() != q.shape[1] or sink.device != dev:
            raise ValueError("sink must be f32 [H] on q's device")
        sink = sink.contiguous()
    T, H, _ = q.shape
    indptr = indptr.contiguous()
    indices = indices.contiguous()
    nnz = indices.numel()
    if out is None:
        out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=dev)
    if return_lse and lse is None:
        lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if ws is None:
        ws = workspace(dev, workspace_bytes(T, H, nnz))
    rc = _lib.sparse_mla_fwd_paged(
        _ptr(q), q.stride(0), q.stride(1),
        desc,
        _ptr(indptr), _ptr(indices) if nnz else None, nnz,
        T, H, float(sm_scale), 1 if has_invalid else 0,
        _ptr(sink),
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse),
        _ptr(ws), ws.numel(),
        _stream(dev))
    _check(rc)
    return out, lse


def _pool_descs(pools, dev):
    if len(pools) != 2:
        raise ValueError("pools must hold two (bytes, page_stride, page_records) triples")
    desc = (KvPool * 2)()
    for i, pl in enumerate(pools):
        buf, stride, per_page = pl
        if buf is None:
            desc[i] = KvPool(None, 0, 0)
            continue
        if buf.dtype != torch.uint8 or buf.dim() != 1 or not buf.is_contiguous() or buf.device != dev:
            raise ValueError("a pool's bytes must be a contiguous 1-D uint8 tensor on q's device")
        desc[i] = KvPool(buf.data_ptr(), int(stride), int(per_page))
    return desc


def v41_workspace_bytes(T: int, H: int, nnz: int) -> int:
    n = int(_lib.sparse_mla_v41_workspace_bytes(int(T), int(H), int(nnz)))
    if n < 0:
        _check(n)
    return n


def fwd_v41(q: torch.Tensor, pools, indptr: torch.Tensor, indices: torch.Tensor, sm_scale: float,
            pos: torch.Tensor, cos_sin: torch.Tensor, sink: Optional[torch.Tensor] = None,
            has_invalid: bool = False, return_lse: bool = True, return_y: bool = False,
            ws: Optional[torch.Tensor] = None):
    """Attention over V4.1 keys (two paged pools: per page, R x 576 data bytes
    then R x 8 scale bytes) with the fused epilogue (bf16, inverse GPT-J
    rotation of dims 448.. at pos[r], MXFP8 of every 32 dims).
    q bf16 [T, H <= 16, 512]; pos int32 [T]; cos_sin f32 [P, 64].
    Returns (xo uint8 [T, H, 512] E4M3 codes, xos uint8 [T, H, 16] E8M0 bytes,
    lse f32 [T, H] or None), plus y f32 [T, H, 512] (the values quantised)
    when return_y."""
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != 512 or q.stride(2) != 1:
        raise ValueError("q must be bf16 [T, H, 512] with contiguous rows")
    if indptr.dtype != torch.int32 or indices.dtype != torch.int32:
        raise ValueError("indptr and indices must be int32")
    dev = q.device
    T, H, _ = q.shape
    if indptr.numel() != T + 1:
        raise ValueError("indptr must have T + 1 entries")
    if pos.dtype != torch.int32 or pos.numel() != T or pos.device != dev:
        raise ValueError("pos must be int32 [T] on q's device")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != 64 or cos_sin.device != dev:
        raise ValueError("cos_sin must be f32 [P, 64] on q's device")
    desc = _pool_descs(pools, dev)
    if sink is not None:
        if sink.dtype != torch.float32 or sink.numel() != H or sink.device != dev:
            raise ValueError("sink must be f32 [H] on q's device")
        sink = sink.contiguous()
    indptr = indptr.contiguous()
    indices = indices.contiguous()
    pos = pos.contiguous()
    cos_sin = cos_sin.contiguous()
    nnz = indices.numel()
    xo = torch.empty(T, H, 512, dtype=torch.uint8, device=dev)
    xos = torch.empty(T, H, 16, dtype=torch.uint8, device=dev)
    lse = torch.empty(T, H, dtype=torch.float32, device=dev) if return_lse else None
    y = torch.empty(T, H, 512, dtype=torch.float32, device=dev) if return_y else None
    if ws is None:
        ws = workspace(dev, v41_workspace_bytes(T, H, nnz))
    _check(_lib.sparse_mla_fwd_v41(
        _ptr(q), q.stride(0), q.stride(1), desc,
        _ptr(indptr), _ptr(indices) if nnz else None, nnz,
        T, H, float(sm_scale), 1 if has_invalid else 0,
        _ptr(sink), _ptr(pos), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(xo), _ptr(xos), _ptr(lse), _ptr(y),
        _ptr(ws), ws.numel(), _stream(dev)))
    return (xo, xos, lse, y) if return_y else (xo, xos, lse)


def mxfp8(y: torch.Tensor):
    """Test hook: the epilogue's MXFP8 quantiser on f32 y [n] (n % 64 == 0)
    -> (codes uint8 [n], E8M0 bytes uint8 [n / 32])."""
    if y.dtype != torch.float32 or y.dim() != 1 or y.numel() % 64:
        raise ValueError("y must be f32 [n] with n a multiple of 64")
    y = y.contiguous()
    codes = torch.empty(y.numel(), dtype=torch.uint8, device=y.device)
    scales = torch.empty(y.numel() // 32, dtype=torch.uint8, device=y.device)
    _check(_lib.sparse_mla_mxfp8(_ptr(y), y.numel(), _ptr(codes), _ptr(scales), _stream(y.device)))
    return codes, scales


def cache_write(latent: torch.Tensor, rope: torch.Tensor, slots: torch.Tensor, kv: torch.Tensor) -> torch.Tensor:
    """Write records kv[slots[i]] from bf16 latent [n, 512] and rope [n, 64]
    (fp8_ds_mla writer rule); slots int64 [n], negative = skip.  Returns kv."""
    if latent.dtype != torch.bfloat16 or latent.dim() != 2 or latent.shape[1] != 512:
        raise ValueError("latent must be bf16 [n, 512]")
    if rope.dtype != torch.bfloat16 or rope.dim() != 2 or rope.shape != (latent.shape[0], 64):
        raise ValueError("rope must be bf16 [n, 64]")
    if latent.stride(1) != 1 or rope.stride(1) != 1:
        raise ValueError("latent and rope rows must be contiguous")
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != RECORD_BYTES or not kv.is_contiguous():
        raise ValueError(f"kv must be contiguous uint8 [N, {RECORD_BYTES}]")
    slots = slots.to(torch.int64).contiguous()
    if slots.numel() != latent.shape[0]:
        raise ValueError("slots must have one entry per token")
    for t in (rope, slots, kv):
        if t.device != latent.device:
            raise ValueError("all tensors must be on latent's device")
    _check(_lib.sparse_mla_cache_write(_ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0),
                                       _ptr(slots), slots.numel(), _ptr(kv), kv.shape[0],
                                       _stream(latent.device)))
    return kv


def decode_rows(kv: torch.Tensor, rows: torch.Tensor) -> torch.Tensor:
    """Decode records kv[rows] to f32 [n, 576] on the device (test hook)."""
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != RECORD_BYTES or not kv.is_contiguous():
        raise ValueError(f"kv must be contiguous uint8 [N, {RECORD_BYTES}]")
    rows = rows.to(torch.int32).contiguous()
    out = torch.empty(rows.numel(), 576, dtype=torch.float32, device=kv.device)
    _check(_lib.sparse_mla_decode_rows(_ptr(kv), kv.shape[0], _ptr(rows), rows.numel(),
                                       _ptr(out), _stream(kv.device)))
    return out


def qk_probe(q16: torch.Tensor, kv: torch.Tensor, rows: torch.Tensor, mode: int) -> torch.Tensor:
    """QK dot products (no sm_scale) of tokens kv[rows] against 16 heads of q
    (bf16 [16, 576]) as f32 [n, 16] (test hook): mode 0 the forward's bf16
    path, 1 the scaled fp8 MFMA with the q hi/lo split (lo = 32 x residual),
    2 its hi part only, 3 the split with lo = 16 x residual."""
    if q16.dtype != torch.bfloat16 or tuple(q16.shape) != (16, 576) or not q16.is_contiguous():
        raise ValueError("q16 must be contiguous bf16 [16, 576]")
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != RECORD_BYTES or not kv.is_contiguous():
        raise ValueError(f"kv must be contiguous uint8 [N, {RECORD_BYTES}]")
    rows = rows.to(torch.int32).contiguous()
    out = torch.empty(rows.numel(), 16, dtype=torch.float32, device=kv.device)
    _check(_lib.sparse_mla_qk_probe(_ptr(q16), _ptr(kv), kv.shape[0], _ptr(rows), rows.numel(), int(mode),
                                    _ptr(out), _stream(kv.device)))
    return out


class KernelTimer:
    """HIP-event timing of the library's kernels over the calls made inside
    the ``with`` block: ``.ms`` and ``.launches`` per kind (plan, fwd, combine,
    cache_write)."""

    KINDS = ("plan", "fwd", "combine", "cache_write")

    def __init__(self, max_calls: int):
        self.max_calls = max_calls
        self.ms = {}
        self.launches = {}

    def __enter__(self):
        _check(_lib.sparse_mla_profile_begin(int(self.max_calls)))
        return self

    def __exit__(self, *exc):
        ms = (ctypes.c_double * len(self.KINDS))()
        n = (_i64 * len(self.KINDS))()
        _check(_lib.sparse_mla_profile_end(ms, n))
        self.ms = {k: ms[i] for i, k in enumerate(self.KINDS)}
        self.launches = {k: int(n[i]) for i, k in enumerate(self.KINDS)}
        return False
