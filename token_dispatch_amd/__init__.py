"""Python binding of libmoonep.so: the balanced expert-parallel hot path on MI355X.

Argument marshalling only. Every step of the plan, dispatch, replicate, combine
and reduce runs in the HIP kernels of the library; torch provides device memory
and streams. The functions carry the C names and take the same arguments:
`dims` is a Dims, arrays are torch tensors on the GPU, `stream` is a
torch.cuda.Stream (default: the current stream of the tensors' device).

If the library has not been built this module raises ImportError: there is no
other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoonep.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' from the repository root)")

_lib = ctypes.CDLL(LIB_PATH)

F32 = 0
BF16 = 1
STATIC_SCRATCH_BYTES = 8 << 20  # MOONEP_STATIC_SCRATCH_BYTES
OK, ERR_DIMS, ERR_PTR, ERR_HIP, ERR_SIZE = 0, -1, -2, -3, -4
STATUS_BAD_ID, STATUS_REPEAT_ID, STATUS_OVER_B = 1, 2, 4
OP_DISPATCH, OP_COMBINE = 1, 2
PLAN_BOUNDED, PLAN_FOUR_LAUNCH, PLAN_TWO_LAUNCH = 1, 2, 4

ENTRY_POINTS = ("moonep_plan_layout", "moonep_plan", "moonep_plan_ex", "moonep_plan_bounded",
                "moonep_plan_noscratch", "moonep_dispatch", "moonep_replicate",
                "moonep_combine", "moonep_reduce_dup_grads", "moonep_combine_backward",
                "moonep_dispatch_backward", "moonep_launch_count", "moonep_strerror")


class Dims(ctypes.Structure):
    """moonep_dims: R ranks, E experts, K per token, S tokens per rank, B duplicate
    slots per rank, dtype of hidden rows (F32/BF16), H hidden size."""
    _fields_ = [("R", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("S", ctypes.c_int32), ("B", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("H", ctypes.c_int64)]

    def __repr__(self):
        return (f"Dims(R={self.R}, E={self.E}, K={self.K}, S={self.S}, B={self.B}, "
                f"dtype={self.dtype}, H={self.H})")


_LAYOUT_OFFSETS = ("status", "maxT", "maxvio", "T", "hoff", "L", "keep", "O", "D", "Opre",
                   "Dpre", "dst", "src", "n_dup", "dup_expert", "dup_start", "dup_count",
                   "seg_ptr", "seg_expert", "n_list", "list_expert", "list_rank", "list_b",
                   "dup_ptr", "ws_tile_counts", "ws_tile_status", "ws_mat_pre", "ws_xlist",
                   "ws_n_x", "ws_piece_js", "ws_kept", "ws_koff", "ws_upre", "ws_pslot",
                   "ws_pcnt")


class Layout(ctypes.Structure):
    _fields_ = ([("bytes", ctypes.c_int64), ("persist_bytes", ctypes.c_int64),
                 ("dcap", ctypes.c_int32), ("pcap", ctypes.c_int32),
                 ("n_tiles", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                 ("plan_launches", ctypes.c_int32)]
                + [(n, ctypes.c_int64) for n in _LAYOUT_OFFSETS])


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_P_DIMS, _P_LAY = ctypes.POINTER(Dims), ctypes.POINTER(Layout)
_lib.moonep_plan_layout.argtypes = [_P_DIMS, _P_LAY]
_lib.moonep_plan.argtypes = [_P_DIMS, _vp, _vp, _vp]
_lib.moonep_plan_bounded.argtypes = [_P_DIMS, _vp, _vp, _vp]
_lib.moonep_plan_ex.argtypes = [_P_DIMS, _vp, _vp, _i32, _vp]
_lib.moonep_plan_noscratch.argtypes = [_P_DIMS, _vp, _vp, _i32, _vp]
_lib.moonep_dispatch.argtypes = [_P_DIMS, _vp, _vp, _vp, _vp]
_lib.moonep_replicate.argtypes = [_P_DIMS, _vp, _vp, _vp, _i64, _vp]
_lib.moonep_combine.argtypes = [_P_DIMS, _vp, _vp, _vp, _vp, _i32, _vp]
_lib.moonep_reduce_dup_grads.argtypes = [_P_DIMS, _vp, _vp, _vp, _i64, _vp]
_lib.moonep_combine_backward.argtypes = [_P_DIMS, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.moonep_dispatch_backward.argtypes = [_P_DIMS, _vp, _vp, _vp, _i32, _vp]
_lib.moonep_launch_count.argtypes = [_P_DIMS, _i32, ctypes.POINTER(ctypes.c_int32)]
_lib.moonep_strerror.argtypes = [ctypes.c_int]
_lib.moonep_strerror.restype = ctypes.c_char_p
for _n in ENTRY_POINTS[:-1]:
    getattr(_lib, _n).restype = ctypes.c_int


class MoonEPError(RuntimeError):
    def __init__(self, rc: int, where: str):
        super().__init__(f"{where}: {moonep_strerror(rc)} (rc={rc})")
        self.rc = rc


def moonep_strerror(rc: int) -> str:
    return _lib.moonep_strerror(rc).decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise MoonEPError(rc, where)


def _torch():
    import torch
    return torch


def _ptr(t, name: str, dtype=None, numel: Optional[int] = None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() * t.element_size() < numel:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {numel}")
    return t.data_ptr()


def _stream(stream, ref) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return stream.cuda_stream


def _row_dtype(dims: Dims):
    torch = _torch()
    return torch.bfloat16 if dims.dtype == BF16 else torch.float32


def moonep_plan_layout(dims: Dims) -> Layout:
    lay = Layout()
    _check(_lib.moonep_plan_layout(ctypes.byref(dims), ctypes.byref(lay)), "moonep_plan_layout")
    return lay


def moonep_launch_count(dims: Dims, op: int) -> int:
    """Kernel launches one moonep_dispatch (OP_DISPATCH) or moonep_combine
    (OP_COMBINE, output in dims.dtype) call enqueues on the current device."""
    n = ctypes.c_int32(0)
    _check(_lib.moonep_launch_count(ctypes.byref(dims), op, ctypes.byref(n)), "moonep_launch_count")
    return int(n.value)


def moonep_plan(dims: Dims, topk_ids, plan_buf, stream=None) -> None:
    torch = _torch()
    lay = moonep_plan_layout(dims)
    ids = _ptr(topk_ids, "topk_ids", torch.int32, 4 * dims.R * dims.S * dims.K)
    pb = _ptr(plan_buf, "plan_buf", None, lay.bytes)
    _check(_lib.moonep_plan(ctypes.byref(dims), ids, pb, _stream(stream, plan_buf)), "moonep_plan")


def moonep_plan_bounded(dims: Dims, topk_ids, plan_buf, stream=None) -> None:
    torch = _torch()
    lay = moonep_plan_layout(dims)
    ids = _ptr(topk_ids, "topk_ids", torch.int32, 4 * dims.R * dims.S * dims.K)
    pb = _ptr(plan_buf, "plan_buf", None, lay.bytes)
    _check(_lib.moonep_plan_bounded(ctypes.byref(dims), ids, pb, _stream(stream, plan_buf)),
           "moonep_plan_bounded")


def moonep_plan_ex(dims: Dims, topk_ids, plan_buf, flags: int = 0, stream=None) -> None:
    """moonep_plan with options: PLAN_BOUNDED, PLAN_FOUR_LAUNCH, PLAN_TWO_LAUNCH."""
    torch = _torch()
    lay = moonep_plan_layout(dims)
    ids = _ptr(topk_ids, "topk_ids", torch.int32, 4 * dims.R * dims.S * dims.K)
    pb = _ptr(plan_buf, "plan_buf", None, lay.bytes)
    _check(_lib.moonep_plan_ex(ctypes.byref(dims), ids, pb, int(flags), _stream(stream, plan_buf)),
           "moonep_plan_ex")


def moonep_plan_noscratch(dims: Dims, topk_ids, plan_buf, bounded: bool = False,
                          stream=None) -> None:
    """moonep_plan (or moonep_plan_bounded) with the plan kernels' scratch in the
    library's static device array: plan_buf needs only persist_bytes bytes."""
    torch = _torch()
    lay = moonep_plan_layout(dims)
    ids = _ptr(topk_ids, "topk_ids", torch.int32, 4 * dims.R * dims.S * dims.K)
    pb = _ptr(plan_buf, "plan_buf", None, lay.persist_bytes)
    _check(_lib.moonep_plan_noscratch(ctypes.byref(dims), ids, pb, 1 if bounded else 0,
                                      _stream(stream, plan_buf)), "moonep_plan_noscratch")


def moonep_dispatch(dims: Dims, plan_buf, hidden, recv, stream=None) -> None:
    dt = _row_dtype(dims)
    row = dims.H * (2 if dims.dtype == BF16 else 4)
    lay = moonep_plan_layout(dims)
    _check(_lib.moonep_dispatch(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(hidden, "hidden", dt, dims.R * dims.S * row),
        _ptr(recv, "recv", dt, dims.R * dims.S * dims.K * row),
        _stream(stream, recv)), "moonep_dispatch")


def moonep_replicate(dims: Dims, plan_buf, expert_w, dup_w, block_bytes: int, stream=None) -> None:
    lay = moonep_plan_layout(dims)
    _check(_lib.moonep_replicate(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(expert_w, "expert_w", None, dims.E * block_bytes),
        _ptr(dup_w, "dup_w", None, dims.R * dims.B * block_bytes),
        int(block_bytes), _stream(stream, dup_w)), "moonep_replicate")


def moonep_combine(dims: Dims, plan_buf, y, topk_w, out, out_dtype: Optional[int] = None,
                   stream=None) -> None:
    torch = _torch()
    od = dims.dtype if out_dtype is None else int(out_dtype)
    row = dims.H * (2 if dims.dtype == BF16 else 4)
    orow = dims.H * (2 if od == BF16 else 4)
    lay = moonep_plan_layout(dims)
    _check(_lib.moonep_combine(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(y, "y", _row_dtype(dims), dims.R * dims.S * dims.K * row),
        _ptr(topk_w, "topk_w", torch.float32, 4 * dims.R * dims.S * dims.K),
        _ptr(out, "out", torch.bfloat16 if od == BF16 else torch.float32, dims.R * dims.S * orow),
        od, _stream(stream, out)), "moonep_combine")


def moonep_reduce_dup_grads(dims: Dims, plan_buf, dup_grads, home_grads, block_elems: int,
                            stream=None) -> None:
    torch = _torch()
    lay = moonep_plan_layout(dims)
    _check(_lib.moonep_reduce_dup_grads(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(dup_grads, "dup_grads", torch.float32, 4 * dims.R * dims.B * block_elems),
        _ptr(home_grads, "home_grads", torch.float32, 4 * dims.E * block_elems),
        int(block_elems), _stream(stream, home_grads)), "moonep_reduce_dup_grads")


def moonep_combine_backward(dims: Dims, plan_buf, grad_out, topk_w, y, grad_y, grad_w,
                            stream=None) -> None:
    """grad_out's dtype (float32 or bfloat16) is passed as gout_dtype; grad_y or
    grad_w may be None to skip that output (then topk_w or y may be None)."""
    torch = _torch()
    g_dt = BF16 if grad_out.dtype == torch.bfloat16 else F32
    grow = dims.H * (2 if g_dt == BF16 else 4)
    row = dims.H * (2 if dims.dtype == BF16 else 4)
    n_ent = dims.R * dims.S * dims.K
    lay = moonep_plan_layout(dims)
    ref = grad_y if grad_y is not None else grad_out
    _check(_lib.moonep_combine_backward(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(grad_out, "grad_out", None, dims.R * dims.S * grow), g_dt,
        None if grad_y is None else _ptr(topk_w, "topk_w", torch.float32, 4 * n_ent),
        None if grad_w is None else _ptr(y, "y", _row_dtype(dims), n_ent * row),
        None if grad_y is None else _ptr(grad_y, "grad_y", _row_dtype(dims), n_ent * row),
        None if grad_w is None else _ptr(grad_w, "grad_w", torch.float32, 4 * n_ent),
        _stream(stream, ref)), "moonep_combine_backward")


def moonep_dispatch_backward(dims: Dims, plan_buf, grad_recv, grad_hidden,
                             out_dtype: Optional[int] = None, stream=None) -> None:
    torch = _torch()
    od = dims.dtype if out_dtype is None else int(out_dtype)
    row = dims.H * (2 if dims.dtype == BF16 else 4)
    orow = dims.H * (2 if od == BF16 else 4)
    lay = moonep_plan_layout(dims)
    _check(_lib.moonep_dispatch_backward(
        ctypes.byref(dims), _ptr(plan_buf, "plan_buf", None, lay.persist_bytes),
        _ptr(grad_recv, "grad_recv", _row_dtype(dims), dims.R * dims.S * dims.K * row),
        _ptr(grad_hidden, "grad_hidden", torch.bfloat16 if od == BF16 else torch.float32,
             dims.R * dims.S * orow), od, _stream(stream, grad_hidden)), "moonep_dispatch_backward")


# ------------------------------------------------------------- buffer helpers

def dims_of(R: int, E: int, K: int, S: int, B: int, H: int, dtype: int) -> Dims:
    return Dims(R, E, K, S, B, dtype, H)


def new_plan_buffer(dims: Dims, device="cuda", persistent_only: bool = False):
    """A device buffer of the size the plan layout asks for (persistent_only: only
    the part that outlives the plan call, enough for moonep_plan_noscratch)."""
    torch = _torch()
    lay = moonep_plan_layout(dims)
    n = lay.persist_bytes if persistent_only else lay.bytes
    return torch.empty(n, dtype=torch.uint8, device=device)


def plan_views(dims: Dims, plan_buf) -> Dict[str, "torch.Tensor"]:
    """Typed views of the public plan arrays inside plan_buf (no copies)."""
    torch = _torch()
    lay = moonep_plan_layout(dims)
    R, E, S, K = dims.R, dims.E, dims.S, dims.K
    G, NE, dcap, pcap = E // R, R * S * K, lay.dcap, lay.pcap
    shapes = {
        "status": (1,), "maxT": (1,), "T": (E,), "hoff": (E,), "L": (R,), "keep": (R,),
        "O": (R,), "D": (R,), "Opre": (R + 1,), "Dpre": (R + 1,), "dst": (NE,), "src": (NE,),
        "n_dup": (R,), "dup_expert": (R, dcap), "dup_start": (R, dcap), "dup_count": (R, dcap),
        "seg_ptr": (R, G + dcap + 1), "seg_expert": (R, G + dcap), "n_list": (1,),
        "list_expert": (pcap,), "list_rank": (pcap,), "list_b": (pcap,), "dup_ptr": (E + 1,),
    }
    out = {}
    for name, shp in shapes.items():
        off = getattr(lay, name)
        n = 1
        for s in shp:
            n *= s
        out[name] = plan_buf[off:off + 4 * n].view(torch.int32).view(shp)
    out["maxvio"] = plan_buf[lay.maxvio:lay.maxvio + 8].view(torch.float64)
    return out
