"""Python binding of libwal (include/wal.h): argument marshalling only.

Every step of a product runs in the HIP kernels of ``libwal.so``; this module
converts numpy arrays and torch tensors to pointers and sizes, passes torch's
current HIP stream, and raises ``WalError`` on a negative status.  torch is
used for device memory and streams only.  If the library is missing the
import fails: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwal.so")

WAL_TRIT_2BIT, WAL_TRIT_BASE3 = 0, 1
WAL_SCALE_FP16, WAL_SCALE_FP24 = 0, 1
WAL_X_F32, WAL_X_BF16 = 0, 1
WAL_X_ROT_H128 = 16   # x_dtype flag: the product rotates x by the normalised H128 first
WAL_GEMM_AUTO, WAL_GEMM_VALU, WAL_GEMM_MFMA = 0, 1, 2
WAL_PHASE_LOWRANK, WAL_PHASE_STREAM, WAL_PHASE_ALL = 1, 2, 3
WAL_MAX_PATHS = 4
WAL_MAX_BATCH = 32
WAL_MAX_PREFILL_BATCH = 16384
WAL_SYNC_BYTES = 4352
WAL_MAX_ROW_BLOCKS = 4096
WAL_WS_ZERO_BYTES = WAL_SYNC_BYTES + 4 * WAL_MAX_ROW_BLOCKS
WAL_SYNC_FALLBACK_WORD = 0

STATUS = {0: "WAL_OK", -1: "WAL_ERR_ARG", -2: "WAL_ERR_SHAPE", -3: "WAL_ERR_CODE",
          -4: "WAL_ERR_INEXACT", -5: "WAL_ERR_BUFFER", -6: "WAL_ERR_ALIGN", -7: "WAL_ERR_FORMAT",
          -8: "WAL_ERR_DEVICE", -9: "WAL_ERR_UNSUPPORTED"}


class WalError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class wal_desc(ctypes.Structure):
    _fields_ = [("out", ctypes.c_uint32), ("in_", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("n_paths", ctypes.c_uint32), ("rank", ctypes.c_uint32),
                ("trit_fmt", ctypes.c_uint32), ("scale_fmt", ctypes.c_uint32)]


class wal_info(ctypes.Structure):
    _fields_ = [("d", wal_desc), ("row_stride", ctypes.c_uint32), ("groups", ctypes.c_uint32),
                ("total_bytes", ctypes.c_uint64), ("off_codes", ctypes.c_uint64),
                ("off_sites", ctypes.c_uint64), ("off_alpha", ctypes.c_uint64),
                ("off_beta", ctypes.c_uint64), ("off_V", ctypes.c_uint64 * 4),
                ("off_U", ctypes.c_uint64 * 4), ("off_s", ctypes.c_uint64 * 4),
                ("algorithmic_bytes", ctypes.c_uint64)]


WAL_MAX_CLASSES = 16


class wal_grouped_info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint32), ("n_classes", ctypes.c_uint32), ("n_segs", ctypes.c_uint32),
                ("n_zjobs", ctypes.c_uint32), ("x_dtype", ctypes.c_uint32), ("zjob_terms", ctypes.c_uint32),
                ("rows_per_batch", ctypes.c_uint32), ("grid", ctypes.c_uint32),
                ("plan_bytes", ctypes.c_uint64), ("algorithmic_bytes", ctypes.c_uint64),
                ("off_descs", ctypes.c_uint64), ("off_zjobs", ctypes.c_uint64),
                ("class_id", ctypes.c_uint32 * WAL_MAX_CLASSES), ("class_grid", ctypes.c_uint32 * WAL_MAX_CLASSES),
                ("class_blockseg", ctypes.c_uint64 * WAL_MAX_CLASSES),
                ("class_segs", ctypes.c_uint64 * WAL_MAX_CLASSES), ("sync_dev", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libwal.so is not built ({LIB_PATH}); run python ternary_hybrid_bit_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_sig = {
    "wal_status_str": (ctypes.c_char_p, [_I]),
    "wal_packed_size": (_I, [ctypes.POINTER(wal_desc), ctypes.POINTER(wal_info)]),
    "wal_pack": (_I, [ctypes.POINTER(wal_desc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                      ctypes.POINTER(wal_info)]),
    "wal_inspect": (_I, [_P, _SZ, ctypes.POINTER(wal_info)]),
    "wal_verify": (_I, [_P, _SZ]),
    "wal_unpack": (_I, [_P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P]),
    "wal_workspace_size": (_I, [ctypes.POINTER(wal_info), _U32, ctypes.POINTER(_SZ)]),
    "wal_gemv": (_I, [ctypes.POINTER(wal_info), _P, _P, _I, _P, _P, _SZ, _P]),
    "wal_gemv_noalloc": (_I, [ctypes.POINTER(wal_info), _P, _P, _I, _P, _P]),
    "wal_gemm_small": (_I, [ctypes.POINTER(wal_info), _P, _P, _I, _U32, _U32, _P, _U32, _I, _P, _SZ, _P]),
    "wal_prefill_workspace_size": (_I, [ctypes.POINTER(wal_info), _U32, ctypes.POINTER(_SZ)]),
    "wal_gemm_prefill": (_I, [ctypes.POINTER(wal_info), _P, _P, _I, _U32, _U32, _P, _U32, _P, _SZ, _P]),
    "wal_grouped_plan_size": (_I, [_U32, _P, _U32, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "wal_grouped_plan": (_I, [_U32, _P, _P, _P, _I, _P, _P, _SZ, _U32, _P, _SZ,
                              ctypes.POINTER(wal_grouped_info)]),
    "wal_gemv_grouped": (_I, [ctypes.POINTER(wal_grouped_info), _P, _P]),
    "wal_gemv_grouped_phases": (_I, [ctypes.POINTER(wal_grouped_info), _P, _I, _P]),
    "wal_rotate_h128": (_I, [_P, _I, _U32, _U32, _U32, _P, _I, _U32, _P]),
    "wal_int4_size": (_I, [_U32, _U32, ctypes.POINTER(_SZ)]),
    "wal_int4_pack": (_I, [_U32, _U32, _P, _P, _P, _SZ]),
    "wal_int4_unpack": (_I, [_U32, _U32, _P, _SZ, _P, _P]),
    "wal_int4_gemv": (_I, [_P, _U32, _U32, _P, _I, _P, _P]),
    "wal_int3_size": (_I, [_U32, _U32, ctypes.POINTER(_SZ)]),
    "wal_int3_pack": (_I, [_U32, _U32, _P, _P, _P, _SZ]),
    "wal_int3_unpack": (_I, [_U32, _U32, _P, _SZ, _P, _P]),
    "wal_embed_rows": (_I, [_P, _I, _U32, _U32, _P, _U32, _P, _I, _U32, _P]),
    "wal_embed_rows_mixed": (_I, [_P, _U32, _P, _U32, _U32, _P, _U32, _P, _U32, _P, _I, _U32, _P]),
    "wal_int5_size": (_I, [_U32, _U32, ctypes.POINTER(_SZ)]),
    "wal_int5_pack": (_I, [_U32, _U32, _P, _P, _P, _SZ]),
    "wal_int5_unpack": (_I, [_U32, _U32, _P, _SZ, _P, _P]),
    "wal_int5_gemv": (_I, [_P, _U32, _U32, _P, _I, _P, _P]),
    "wal_gemv_grouped_seq": (_I, [_U32, _P, _P, _P]),
    "wal_graph_create": (_I, [_U32, _P, _P, ctypes.POINTER(_P)]),
    "wal_graph_launch": (_I, [_P, _P]),
    "wal_graph_destroy": (_I, [_P]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(st: int, where: str):
    if st != 0:
        raise WalError(st, where)


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()  # torch tensor


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# Checks of device arguments.  The C ABI takes bare pointers and cannot see a
# buffer's size, dtype or device, so the binding checks them before any call:
# a wrong dtype or a short buffer would otherwise become out-of-bounds device
# reads or writes.  Type, dtype, shape and size are checked before the device,
# so every check can be exercised on CPU tensors.

def _torch():
    import torch
    return torch


def _dev(t, name: str, dtypes, min_numel: int = 0):
    """t must be a torch tensor of one of ``dtypes`` (torch dtypes), with at
    least ``min_numel`` elements and unit stride along its last axis."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor on the GPU, not {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {[str(d) for d in dtypes]}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements; at least {min_numel} are needed")
    if t.dim() > 0 and t.numel() > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride along its last axis")
    if t.dim() > 2:
        raise ValueError(f"{name} must be 1-D or 2-D")
    return t


def _dev_bytes(t, name: str, min_bytes: int):
    """A byte buffer (any dtype) of at least min_bytes bytes, contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor on the GPU, not {type(t).__name__}")
    nb = t.numel() * t.element_size()
    if nb < min_bytes:
        raise ValueError(f"{name} holds {nb} bytes; at least {min_bytes} are needed")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _gpu(**tensors):
    """Every named tensor (None skipped) must live on a GPU; checked after
    all other checks of a call."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU (device {t.device})")


def _xdtype(t) -> int:
    torch = _torch()
    return WAL_X_BF16 if t.dtype == torch.bfloat16 else WAL_X_F32


def _act(t, name: str, n: int):
    """An activation vector: bf16 or fp32, at least n elements."""
    torch = _torch()
    return _dev(t, name, (torch.bfloat16, torch.float32), n)


def _rows(t, name: str, dtypes, cols: int, rows: Optional[int] = None):
    """A 2-D [rows][ld] device matrix with ld >= cols (unit column stride)."""
    _dev(t, name, dtypes)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows][ld]")
    if t.shape[1] < cols:
        raise ValueError(f"{name} has {t.shape[1]} columns; at least {cols} are needed")
    if rows is not None and t.shape[0] < rows:
        raise ValueError(f"{name} has {t.shape[0]} rows; at least {rows} are needed")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows overlap (stride {t.stride(0)} < {t.shape[1]})")
    return t


def _ws_bytes(ws, name: str = "ws") -> int:
    """Byte size of a workspace tensor (0 for None); the library checks it
    against what the product needs."""
    if ws is None:
        return 0
    _dev_bytes(ws, name, 0)
    return ws.numel() * ws.element_size()


def sync_fallbacks(ws) -> int:
    """The fallback count of a workspace's synchronisation words: the
    workgroups of earlier calls whose bounded wait for the low-rank terms
    gave up and which computed the terms themselves.  Synchronises the
    device."""
    words = ws.view(-1).view(_torch().uint8)[:WAL_SYNC_BYTES].view(_torch().int32)
    return int(words[WAL_SYNC_FALLBACK_WORD].item())


def clear_sync_fallbacks(ws):
    """Clears that count (on the current stream)."""
    words = ws.view(-1).view(_torch().uint8)[:WAL_SYNC_BYTES].view(_torch().int32)
    words[WAL_SYNC_FALLBACK_WORD] = 0


def wal_status_str(status: int) -> str:
    return _lib.wal_status_str(status).decode()


def make_desc(out, inp, k=8, n_paths=0, rank=0, trit_fmt=WAL_TRIT_2BIT, scale_fmt=WAL_SCALE_FP16) -> wal_desc:
    return wal_desc(out, inp, k, n_paths, rank if n_paths else 0, trit_fmt, scale_fmt)


def wal_packed_size(desc: wal_desc) -> wal_info:
    info = wal_info()
    _check(_lib.wal_packed_size(ctypes.byref(desc), ctypes.byref(info)), "wal_packed_size")
    return info


def wal_pack(desc: wal_desc, T, site_pos=None, site_sign=None, alpha=None, beta=None,
             U=None, V=None, s=None):
    """Pack logical arrays (numpy) into a new uint8 blob; returns (blob, info)."""
    info = wal_packed_size(desc)
    dst = np.zeros(info.total_bytes, dtype=np.uint8)
    arrays = [_c(T, np.int8), _c(site_pos, np.uint8), _c(site_sign, np.int8), _c(alpha, np.float32),
              _c(beta, np.float32), _c(U, np.int8), _c(V, np.int8), _c(s, np.float32)]
    out = wal_info()
    st = _lib.wal_pack(ctypes.byref(desc), *[_ptr(a) for a in arrays], dst.ctypes.data, dst.size,
                       ctypes.byref(out))
    _check(st, "wal_pack")
    return dst, out


def pack_matrix(m) -> tuple:
    """Pack a ``synth.Matrix``-like object (fields T, site_pos, ...)."""
    desc = make_desc(m.out, m.inp, m.k, m.U.shape[0], m.U.shape[2] if m.U.shape[0] else 0,
                     m.trit_fmt, m.scale_fmt)
    k = m.k
    return wal_pack(desc, m.T, m.site_pos if k else None, m.site_sign if k else None, m.alpha,
                    m.beta if k else None, m.U if m.U.shape[0] else None,
                    m.V if m.U.shape[0] else None, m.s if m.U.shape[0] else None)


def wal_inspect(blob) -> wal_info:
    b = np.ascontiguousarray(blob, dtype=np.uint8) if not isinstance(blob, np.ndarray) else blob
    info = wal_info()
    _check(_lib.wal_inspect(b.ctypes.data, b.size, ctypes.byref(info)), "wal_inspect")
    return info


def wal_verify(blob) -> int:
    b = np.frombuffer(blob, dtype=np.uint8) if isinstance(blob, (bytes, bytearray)) else blob
    return _lib.wal_verify(b.ctypes.data, b.size)


def wal_unpack(blob) -> dict:
    b = np.frombuffer(blob, dtype=np.uint8) if isinstance(blob, (bytes, bytearray)) else blob
    info = wal_inspect(b)
    d = info.d
    G = d.in_ // 128
    P, r = d.n_paths, d.rank
    o = {"T": np.zeros((d.out, d.in_), np.int8), "site_pos": np.zeros((d.out, G, d.k), np.uint8),
         "site_sign": np.zeros((d.out, G, d.k), np.int8), "alpha": np.zeros((d.out, G), np.float32),
         "beta": np.zeros((d.out, G), np.float32) if d.k else None,
         "U": np.zeros((P, d.out, r), np.int8), "V": np.zeros((P, d.in_, r), np.int8),
         "s": np.zeros((P, r), np.float32)}
    st = _lib.wal_unpack(b.ctypes.data, b.size, *[_ptr(o[k]) if o[k] is not None and o[k].size else None
                                                   for k in ("T", "site_pos", "site_sign", "alpha", "beta",
                                                             "U", "V", "s")])
    _check(st, "wal_unpack")
    return o


def wal_workspace_size(info: wal_info, batch: int = 1) -> int:
    n = _SZ()
    _check(_lib.wal_workspace_size(ctypes.byref(info), batch, ctypes.byref(n)), "wal_workspace_size")
    return n.value


def wal_prefill_workspace_size(info: wal_info, batch: int) -> int:
    n = _SZ()
    _check(_lib.wal_prefill_workspace_size(ctypes.byref(info), batch, ctypes.byref(n)), "wal_prefill_workspace_size")
    return n.value


def wal_gemv(info: wal_info, W, x, y, ws=None, stream=None, rotate=False):
    """y = W(x) on the GPU; W, x, y (and ws, see wal_workspace_size) are device
    tensors; y is fp32 [out].  rotate: the blob is stored rotated, and the
    launch rotates x by the normalised H128 first (WAL_X_ROT_H128)."""
    torch = _torch()
    _dev_bytes(W, "W", int(info.total_bytes))
    _act(x, "x", int(info.d.in_))
    _dev(y, "y", (torch.float32,), int(info.d.out))
    xdt = _xdtype(x) | (WAL_X_ROT_H128 if rotate else 0)
    wsb = _ws_bytes(ws)
    _gpu(W=W, x=x, y=y, ws=ws)
    st = _lib.wal_gemv(ctypes.byref(info), _ptr(W), _ptr(x), xdt, _ptr(y), _ptr(ws), wsb, _stream(stream))
    _check(st, "wal_gemv")
    return y


def wal_gemv_noalloc(info: wal_info, W, x, y, stream=None, rotate=False):
    """y = W(x) as wal_gemv, with the library's per-device scratch as the
    workspace (nothing is allocated; overlapping calls on one GPU race)."""
    torch = _torch()
    _dev_bytes(W, "W", int(info.total_bytes))
    _act(x, "x", int(info.d.in_))
    _dev(y, "y", (torch.float32,), int(info.d.out))
    _gpu(W=W, x=x, y=y)
    xdt = _xdtype(x) | (WAL_X_ROT_H128 if rotate else 0)
    st = _lib.wal_gemv_noalloc(ctypes.byref(info), _ptr(W), _ptr(x), xdt, _ptr(y), _stream(stream))
    _check(st, "wal_gemv_noalloc")
    return y


def wal_gemm_small(info: wal_info, W, X, Y, mode=WAL_GEMM_AUTO, ws=None, stream=None):
    """Y = X W^T on the GPU; X [batch][ldx], Y [batch][ldy] device tensors."""
    torch = _torch()
    _dev_bytes(W, "W", int(info.total_bytes))
    _rows(X, "X", (torch.bfloat16, torch.float32), int(info.d.in_))
    _rows(Y, "Y", (torch.float32,), int(info.d.out), X.shape[0])
    xdt = _xdtype(X)
    if not 1 <= X.shape[0] <= WAL_MAX_BATCH:
        raise ValueError(f"batch {X.shape[0]} outside 1..{WAL_MAX_BATCH}")
    wsb = _ws_bytes(ws)
    _gpu(W=W, X=X, Y=Y, ws=ws)
    st = _lib.wal_gemm_small(ctypes.byref(info), _ptr(W), _ptr(X), xdt, X.shape[0], X.stride(0), _ptr(Y),
                             Y.stride(0), mode, _ptr(ws), wsb, _stream(stream))
    _check(st, "wal_gemm_small")
    return Y


def wal_gemm_prefill(info: wal_info, W, X, Y, ws=None, stream=None):
    """Y = X W^T for a prefill-size batch; X [batch][ldx] bf16, Y [batch][ldy]
    fp32 device tensors, ws of wal_prefill_workspace_size bytes (or None when 0)."""
    torch = _torch()
    _dev_bytes(W, "W", int(info.total_bytes))
    _rows(X, "X", (torch.bfloat16, torch.float32), int(info.d.in_))
    _rows(Y, "Y", (torch.float32,), int(info.d.out), X.shape[0])
    xdt = _xdtype(X)
    if not 1 <= X.shape[0] <= WAL_MAX_PREFILL_BATCH:
        raise ValueError(f"batch {X.shape[0]} outside 1..{WAL_MAX_PREFILL_BATCH}")
    wsb = _ws_bytes(ws)
    _gpu(W=W, X=X, Y=Y, ws=ws)
    st = _lib.wal_gemm_prefill(ctypes.byref(info), _ptr(W), _ptr(X), xdt, X.shape[0], X.stride(0), _ptr(Y),
                               Y.stride(0), _ptr(ws), wsb, _stream(stream))
    _check(st, "wal_gemm_prefill")
    return Y


def wal_grouped_plan_size(infos: Sequence[wal_info], grid: int = 0, x_dtype: int = WAL_X_BF16):
    """(plan_bytes, ws_bytes) of a grouped plan; grid 0 = what the current GPU holds at once."""
    arr = (wal_info * len(infos))(*infos)
    pb, wb = _SZ(), _SZ()
    _check(_lib.wal_grouped_plan_size(len(infos), arr, grid, x_dtype, ctypes.byref(pb), ctypes.byref(wb)),
           "wal_grouped_plan_size")
    return pb.value, wb.value


def wal_grouped_plan(infos: Sequence[wal_info], Ws, xs, ys, ws, x_dtype: int, grid: int = 0):
    """Build a grouped plan; returns (plan bytes as numpy uint8, wal_grouped_info).
    x_dtype may carry WAL_X_ROT_H128 (every matrix of the plan rotated)."""
    torch = _torch()
    n = len(infos)
    if not (len(Ws) == len(xs) == len(ys) == n):
        raise ValueError("infos, Ws, xs and ys must have the same length")
    xt = torch.bfloat16 if (x_dtype & ~WAL_X_ROT_H128) == WAL_X_BF16 else torch.float32
    for i, (f, w, x, y) in enumerate(zip(infos, Ws, xs, ys)):
        _dev_bytes(w, f"Ws[{i}]", int(f.total_bytes))
        _dev(x, f"xs[{i}]", (xt,), int(f.d.in_))
        _dev(y, f"ys[{i}]", (torch.float32,), int(f.d.out))
    arr = (wal_info * n)(*infos)
    pb, _ = wal_grouped_plan_size(infos, grid, x_dtype)
    plan = np.zeros(pb, dtype=np.uint8)
    Wp = (ctypes.c_void_p * n)(*[_ptr(w) for w in Ws])
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    g = wal_grouped_info()
    wsb = _ws_bytes(ws)
    for i, (w, x, y) in enumerate(zip(Ws, xs, ys)):
        _gpu(**{f"Ws[{i}]": w, f"xs[{i}]": x, f"ys[{i}]": y})
    _gpu(ws=ws)
    st = _lib.wal_grouped_plan(n, arr, Wp, xp, x_dtype, yp, _ptr(ws), wsb, grid, plan.ctypes.data, plan.size,
                               ctypes.byref(g))
    _check(st, "wal_grouped_plan")
    return plan, g


def _plan(ginfo: wal_grouped_info, plan_dev, name="plan_dev"):
    _dev_bytes(plan_dev, name, int(ginfo.plan_bytes))
    _gpu(**{name: plan_dev})
    return plan_dev


def wal_gemv_grouped(ginfo: wal_grouped_info, plan_dev, stream=None):
    _plan(ginfo, plan_dev)
    _check(_lib.wal_gemv_grouped(ctypes.byref(ginfo), _ptr(plan_dev), _stream(stream)), "wal_gemv_grouped")


def wal_gemv_grouped_phases(ginfo: wal_grouped_info, plan_dev, phases: int, stream=None):
    _plan(ginfo, plan_dev)
    _check(_lib.wal_gemv_grouped_phases(ctypes.byref(ginfo), _ptr(plan_dev), phases, _stream(stream)),
           "wal_gemv_grouped_phases")


def exported_symbols() -> list:
    return list(_sig)


def _chain_args(chain):
    """chain: [(wal_grouped_info, plan device tensor)] -> ctypes arrays."""
    n = len(chain)
    for i, (g, p) in enumerate(chain):
        _plan(g, p, f"chain[{i}] plan")
    infos = (wal_grouped_info * n)(*[g for g, _ in chain])
    plans = (ctypes.c_void_p * n)(*[_ptr(p) for _, p in chain])
    return n, infos, plans


def wal_gemv_grouped_seq(chain, stream=None):
    """Launch the grouped products of ``chain`` in order on the stream."""
    n, infos, plans = _chain_args(chain)
    _check(_lib.wal_gemv_grouped_seq(n, infos, plans, _stream(stream)), "wal_gemv_grouped_seq")


class WalGraph:
    """A chain of grouped products captured in a HIP graph (wal_graph_create);
    launch() replays it on a stream; the buffers the plans name must outlive it."""

    def __init__(self, chain):
        n, infos, plans = _chain_args(chain)
        h = ctypes.c_void_p()
        _check(_lib.wal_graph_create(n, infos, plans, ctypes.byref(h)), "wal_graph_create")
        self._h = h

    def launch(self, stream=None):
        _check(_lib.wal_graph_launch(self._h, _stream(stream)), "wal_graph_launch")

    def close(self):
        if self._h:
            _check(_lib.wal_graph_destroy(self._h), "wal_graph_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass


def wal_rotate_h128(X, out, stream=None):
    """out = X rotated by the normalised Hadamard-128 along its last axis (1-D
    or 2-D device tensors, bf16 or fp32; out may be X itself)."""
    torch = _torch()
    acts = (torch.bfloat16, torch.float32)
    _dev(X, "X", acts)
    _dev(out, "out", acts)
    X2 = X if X.dim() == 2 else X.view(1, -1)
    O2 = out if out.dim() == 2 else out.view(1, -1)
    _rows(O2, "out", acts, X2.shape[1], X2.shape[0])
    _gpu(X=X, out=out)
    dt = _xdtype
    st = _lib.wal_rotate_h128(_ptr(X2), dt(X), X2.shape[0], X2.shape[1], X2.stride(0), _ptr(O2), dt(out),
                              O2.stride(0), _stream(stream))
    _check(st, "wal_rotate_h128")
    return out


def wal_int4_size(V: int, inp: int) -> int:
    n = _SZ()
    _check(_lib.wal_int4_size(V, inp, ctypes.byref(n)), "wal_int4_size")
    return n.value


def wal_int4_pack(q, s) -> np.ndarray:
    """INT4/g128 codes q [V][in] in [-8, 7] and scales s [V][in/128] -> packed bytes (host)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    V, inp = q.shape
    out = np.zeros(wal_int4_size(V, inp), dtype=np.uint8)
    _check(_lib.wal_int4_pack(V, inp, q.ctypes.data, s.ctypes.data, out.ctypes.data, out.size), "wal_int4_pack")
    return out


def wal_int4_unpack(blob: np.ndarray, V: int, inp: int):
    q = np.zeros((V, inp), dtype=np.int8)
    s = np.zeros((V, inp // 128), dtype=np.float32)
    _check(_lib.wal_int4_unpack(V, inp, blob.ctypes.data, blob.size, q.ctypes.data, s.ctypes.data), "wal_int4_unpack")
    return q, s


def wal_int4_gemv(W, V: int, inp: int, x, y, stream=None):
    """y = W x for an INT4/g128 matrix W (device bytes), x [in] bf16, y [V] fp32."""
    torch = _torch()
    _dev_bytes(W, "W", wal_int4_size(V, inp))
    _act(x, "x", inp)
    _dev(y, "y", (torch.float32,), V)
    xdt = _xdtype(x)
    _gpu(W=W, x=x, y=y)
    _check(_lib.wal_int4_gemv(_ptr(W), V, inp, _ptr(x), xdt, _ptr(y), _stream(stream)), "wal_int4_gemv")
    return y


def wal_int3_size(V: int, inp: int) -> int:
    n = _SZ()
    _check(_lib.wal_int3_size(V, inp, ctypes.byref(n)), "wal_int3_size")
    return n.value


def wal_int3_pack(q, s) -> np.ndarray:
    """INT3/g128 codes q [V][in] in [-4, 3] and scales s [V][in/128] -> packed bytes (host)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    V, inp = q.shape
    out = np.zeros(wal_int3_size(V, inp), dtype=np.uint8)
    _check(_lib.wal_int3_pack(V, inp, q.ctypes.data, s.ctypes.data, out.ctypes.data, out.size), "wal_int3_pack")
    return out


def wal_int3_unpack(blob: np.ndarray, V: int, inp: int):
    q = np.zeros((V, inp), dtype=np.int8)
    s = np.zeros((V, inp // 128), dtype=np.float32)
    _check(_lib.wal_int3_unpack(V, inp, blob.ctypes.data, blob.size, q.ctypes.data, s.ctypes.data), "wal_int3_unpack")
    return q, s


def wal_int5_size(V: int, inp: int) -> int:
    n = _SZ()
    _check(_lib.wal_int5_size(V, inp, ctypes.byref(n)), "wal_int5_size")
    return n.value


def wal_int5_pack(q, s) -> np.ndarray:
    """INT5/g128 codes q [V][in] in [-16, 15] and scales s [V][in/128] -> packed bytes (host)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    V, inp = q.shape
    out = np.zeros(wal_int5_size(V, inp), dtype=np.uint8)
    _check(_lib.wal_int5_pack(V, inp, q.ctypes.data, s.ctypes.data, out.ctypes.data, out.size), "wal_int5_pack")
    return out


def wal_int5_unpack(blob: np.ndarray, V: int, inp: int):
    q = np.zeros((V, inp), dtype=np.int8)
    s = np.zeros((V, inp // 128), dtype=np.float32)
    _check(_lib.wal_int5_unpack(V, inp, blob.ctypes.data, blob.size, q.ctypes.data, s.ctypes.data), "wal_int5_unpack")
    return q, s


def wal_int5_gemv(W, V: int, inp: int, x, y, stream=None):
    """y = W x for an INT5/g128 matrix W (device bytes), x [in] bf16, y [V] fp32."""
    torch = _torch()
    _dev_bytes(W, "W", wal_int5_size(V, inp))
    _act(x, "x", inp)
    _dev(y, "y", (torch.float32,), V)
    xdt = _xdtype(x)
    _gpu(W=W, x=x, y=y)
    _check(_lib.wal_int5_gemv(_ptr(W), V, inp, _ptr(x), xdt, _ptr(y), _stream(stream)), "wal_int5_gemv")
    return y


def wal_embed_rows(W, bits: int, V: int, inp: int, ids, out, stream=None):
    """out[i] = row ids[i] of an INT3 (bits 3) or INT4 (bits 4) matrix W (device
    bytes); ids int32 [n] and out [n][ldo] (fp32 or bf16) device tensors."""
    torch = _torch()
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    _dev_bytes(W, "W", wal_int3_size(V, inp) if bits == 3 else wal_int4_size(V, inp))
    _dev(ids, "ids", (torch.int32,))
    _rows(out, "out", (torch.float32, torch.bfloat16), inp, ids.numel())
    odt = _xdtype(out)
    _gpu(W=W, ids=ids, out=out)
    _check(_lib.wal_embed_rows(_ptr(W), bits, V, inp, _ptr(ids), ids.numel(), _ptr(out), odt, out.stride(0),
                               _stream(stream)), "wal_embed_rows")
    return out


def wal_embed_rows_mixed(W3, V3: int, W4, V4: int, inp: int, row_map, ids, out, stream=None):
    """out[i] = vocabulary row ids[i] of a mixed table: row_map[v] >= 0 names
    a row of the INT3 table W3, a negative entry m row -1 - m of the INT4
    table W4 (device bytes); row_map and ids int32, out [n][ldo] device."""
    torch = _torch()
    _dev_bytes(W3, "W3", wal_int3_size(V3, inp) if V3 else 0)
    _dev_bytes(W4, "W4", wal_int4_size(V4, inp) if V4 else 0)
    _dev(row_map, "row_map", (torch.int32,))
    _dev(ids, "ids", (torch.int32,))
    _rows(out, "out", (torch.float32, torch.bfloat16), inp, ids.numel())
    odt = _xdtype(out)
    _gpu(W3=W3, W4=W4, row_map=row_map, ids=ids, out=out)
    _check(_lib.wal_embed_rows_mixed(_ptr(W3), V3, _ptr(W4), V4, inp, _ptr(row_map), row_map.numel(), _ptr(ids),
                                     ids.numel(), _ptr(out), odt, out.stride(0), _stream(stream)),
           "wal_embed_rows_mixed")
    return out

