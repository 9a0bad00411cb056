"""CPU oracle for the balanced expert-parallel plan and its data moves.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg load it; the HIP library never does, and the two share no code.
The arithmetic lives in moonep_oracle.c (plain loops, built with gcc
-O2 -ffp-contract=off -fopenmp; the data moves spread their outer loop over
threads, every output element with one writer, so the thread count never changes
a bit); this module builds it on first use and marshals numpy arrays in and out.
Each function names the passage it follows in its C source.

Parity status of each function (what pins it, see tests/test_oracle_pins.py):
  plan      -- pinned: library histogram, hand-worked examples, an independent
               sort-and-slice formulation on brute-forced tiny inputs, closed-form
               balanced cases, invariants
  dispatch  -- pinned: hand-worked examples (token order of every slot)
  replicate -- pinned: hand-worked example
  combine   -- pinned: closed forms, binary64 error bound, library bf16 rounding
  reduce    -- pinned: hand-derived rounding-order value, integer closed form,
               binary64 error bound
  plan(bounded=True)
            -- pinned: hand-worked examples, invariants of any balanced plan plus
               the B bound, brute-force minimality of the overflowing experts,
               closed forms (balanced input, one overloaded rank)
  combine_backward_y, combine_backward_w, dispatch_backward
            -- pinned: torch autograd in binary64 of the plain forward
               definitions (gather, weighted sum), torch's bf16 rounding, closed
               forms (unit weights, K copies of a bf16 row), binary64 error bounds
tests/test_oracle_mutants.py plants mistakes in copies of the C source and checks
that the pins above reject every one of them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moonep_oracle.c")
_LIB = os.path.join(_HERE, "libmoonep_oracle.so")

F32 = 0
BF16 = 1
ST_BAD_ID, ST_REPEAT_ID, ST_OVER_B = 1, 2, 4


# gcc flags of the oracle (plain C, no contraction of a*b+c; OpenMP for the moves)
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
          "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc"] + CFLAGS + ["-Wall", "-Werror", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.POINTER


class _PlanOut(ctypes.Structure):
    _fields_ = [("status", _P(ctypes.c_int32)), ("maxT", _P(ctypes.c_int64)),
                ("maxvio", _P(ctypes.c_double))] + [
        (n, _P(ctypes.c_int32)) for n in (
            "T", "hoff", "L", "keep", "O", "D", "Opre", "Dpre", "dst", "src", "n_dup",
            "dup_expert", "dup_start", "dup_count", "seg_ptr", "seg_expert", "n_list",
            "list_expert", "list_rank", "list_b", "dup_ptr")]


# Test hook: the mutation test (tests/test_oracle_mutants.py) runs the pins in a
# child process with this variable naming a deliberately broken build of the
# oracle, to show that the pins reject it. Nothing else sets it.
LIB_OVERRIDE_ENV = "MOONEP_ORACLE_LIB"


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get(LIB_OVERRIDE_ENV)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_plan.argtypes = [i32, i32, i32, i32, i32, vp, i32, i32, _P(_PlanOut)]
        lib.oracle_plan.restype = ctypes.c_int
        lib.oracle_plan_bounded.argtypes = [i32, i32, i32, i32, i32, vp, i32, i32, _P(_PlanOut)]
        lib.oracle_plan_bounded.restype = ctypes.c_int
        lib.oracle_dispatch.argtypes = [i64, i32, i64, vp, vp, i64, i64, vp]
        lib.oracle_dispatch.restype = None
        lib.oracle_replicate.argtypes = [i32, i32, i32, vp, vp, i64, vp, vp]
        lib.oracle_replicate.restype = None
        lib.oracle_combine.argtypes = [i64, i32, i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_combine.restype = None
        lib.oracle_reduce.argtypes = [i32, i32, i64, vp, vp, vp, vp, vp]
        lib.oracle_reduce.restype = None
        lib.oracle_f32_to_bf16.argtypes = [i64, vp, vp]
        lib.oracle_f32_to_bf16.restype = None
        lib.oracle_combine_backward_y.argtypes = [i64, i32, i64, i32, i32, vp, vp, vp, i64, i64, vp]
        lib.oracle_combine_backward_y.restype = None
        lib.oracle_combine_backward_w.argtypes = [i64, i32, i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_combine_backward_w.restype = None
        lib.oracle_dispatch_backward.argtypes = [i64, i32, i64, i32, i32, vp, vp, vp]
        lib.oracle_dispatch_backward.restype = None
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_set_threads.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def dcap_of(R: int, E: int, K: int, S: int) -> int:
    """Most duplicates one rank can hold: distinct non-home experts, at most one
    slot each (at least 1, so arrays are never empty)."""
    return max(1, min(S * K, E - E // R))


def pcap_of(R: int, E: int) -> int:
    """Room for the global duplicate list (pieces <= overflowing experts + deficit ranks - 1)."""
    return E + R


def plan(R: int, E: int, K: int, S: int, B: int, ids: np.ndarray,
         bounded: bool = False) -> Dict[str, np.ndarray]:
    """The water-fill plan of one step's router ids [R,S,K] (see moonep_oracle.c);
    bounded=True gives the plan that keeps at most B duplicates per rank where it
    can (oracle_plan_bounded)."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    if ids.size != R * S * K:
        raise ValueError("ids must hold R*S*K entries")
    G = E // R
    dcap, pcap = dcap_of(R, E, K, S), pcap_of(R, E)
    i32 = np.int32
    out = {
        "status": np.zeros(1, i32), "maxT": np.zeros(1, np.int64), "maxvio": np.zeros(1, np.float64),
        "T": np.zeros(E, i32), "hoff": np.zeros(E, i32), "L": np.zeros(R, i32),
        "keep": np.zeros(R, i32), "O": np.zeros(R, i32), "D": np.zeros(R, i32),
        "Opre": np.zeros(R + 1, i32), "Dpre": np.zeros(R + 1, i32),
        "dst": np.zeros(R * S * K, i32), "src": np.zeros(R * S * K, i32),
        "n_dup": np.zeros(R, i32), "dup_expert": np.zeros((R, dcap), i32),
        "dup_start": np.zeros((R, dcap), i32), "dup_count": np.zeros((R, dcap), i32),
        "seg_ptr": np.zeros((R, G + dcap + 1), i32), "seg_expert": np.zeros((R, G + dcap), i32),
        "n_list": np.zeros(1, i32), "list_expert": np.zeros(pcap, i32),
        "list_rank": np.zeros(pcap, i32), "list_b": np.zeros(pcap, i32),
        "dup_ptr": np.zeros(E + 1, i32),
    }
    po = _PlanOut()
    for name, ctype in _PlanOut._fields_:
        setattr(po, name, ctypes.cast(out[name].ctypes.data, ctype))
    fn = lib.oracle_plan_bounded if bounded else lib.oracle_plan
    rc = fn(R, E, K, S, B, _ptr(ids), dcap, pcap, ctypes.byref(po))
    if rc != 0:
        raise ValueError("oracle_plan rejected its arguments")
    out["dcap"], out["pcap"] = dcap, pcap
    return out


def set_threads(n: int) -> None:
    """Threads of the data moves (the plan always runs on one)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def dispatch(plan_out: Dict[str, np.ndarray], K: int, hidden: np.ndarray,
             slot_lo: int = 0, slot_hi: Optional[int] = None,
             out: Optional[np.ndarray] = None) -> np.ndarray:
    """recv rows for slots [slot_lo, slot_hi): bytes of hidden [n_tok, H] (any dtype).
    `out`, if given, receives them (rows of slots holding no entry keep its contents);
    else a zeroed array is returned."""
    lib = _load()
    hidden = np.ascontiguousarray(hidden)
    n_tok = hidden.shape[0]
    row_bytes = hidden.strides[0]
    dst = plan_out["dst"]
    if slot_hi is None:
        slot_hi = dst.size
    shape = (slot_hi - slot_lo,) + hidden.shape[1:]
    if out is None:
        recv = np.zeros(shape, dtype=hidden.dtype)
    else:
        if out.shape != shape or out.dtype != hidden.dtype or not out.flags["C_CONTIGUOUS"]:
            raise ValueError("out must be a contiguous array of the window's shape and dtype")
        recv = out
    lib.oracle_dispatch(dst.size, K, row_bytes, _ptr(hidden), _ptr(dst), slot_lo, slot_hi,
                        _ptr(recv))
    assert n_tok * K == dst.size
    return recv


def replicate(plan_out: Dict[str, np.ndarray], B: int, expert_w: np.ndarray) -> np.ndarray:
    """dup_w [R, B, block...] with slots b < min(n_dup, B) filled; others zero."""
    lib = _load()
    expert_w = np.ascontiguousarray(expert_w)
    R = plan_out["n_dup"].size
    blk = expert_w.strides[0]
    dup_w = np.zeros((R, B) + expert_w.shape[1:], dtype=expert_w.dtype)
    lib.oracle_replicate(R, B, plan_out["dcap"], _ptr(plan_out["n_dup"]),
                         _ptr(plan_out["dup_expert"]), blk, _ptr(expert_w), _ptr(dup_w))
    return dup_w


def combine(dst: np.ndarray, K: int, y: np.ndarray, w: np.ndarray, in_dtype: int,
            out_dtype: int) -> np.ndarray:
    """out [n_tok, H]: y is [n_slots, H] as float32 (F32) or uint16 bf16 bits (BF16);
    dst and w are [n_tok*K]; the result is float32 or uint16 bf16 bits."""
    lib = _load()
    y = np.ascontiguousarray(y)
    dst = np.ascontiguousarray(dst, dtype=np.int32).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    H = y.shape[-1]
    n_tok = dst.size // K
    assert y.dtype == (np.uint16 if in_dtype == BF16 else np.float32)
    out = np.zeros((n_tok, H), dtype=np.uint16 if out_dtype == BF16 else np.float32)
    lib.oracle_combine(n_tok, K, H, in_dtype, out_dtype, _ptr(y), _ptr(dst), _ptr(w), _ptr(out))
    return out


def reduce_dup_grads(plan_out: Dict[str, np.ndarray], B: int, dup_grads: np.ndarray,
                     home_grads: np.ndarray) -> np.ndarray:
    """Returns home_grads [E, n] after adding each expert's duplicate gradients."""
    lib = _load()
    dup = np.ascontiguousarray(dup_grads, dtype=np.float32)
    home = np.array(home_grads, dtype=np.float32, copy=True, order="C")
    E = home.shape[0]
    n = home[0].size
    lib.oracle_reduce(E, B, n, _ptr(plan_out["dup_ptr"]), _ptr(plan_out["list_rank"]),
                      _ptr(plan_out["list_b"]), _ptr(dup), _ptr(home))
    return home


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """The combine's output rounding (binary32 -> bf16 bits, nearest-even)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    y = np.zeros(x.size, dtype=np.uint16)
    lib.oracle_f32_to_bf16(x.size, _ptr(x), _ptr(y))
    return y


def _row_type(dtype: int):
    return np.uint16 if dtype == BF16 else np.float32


def combine_backward_y(dst: np.ndarray, K: int, grad_out: np.ndarray, w: np.ndarray,
                       gout_dtype: int, y_dtype: int, slot_lo: int = 0,
                       slot_hi: Optional[int] = None, fill=0) -> np.ndarray:
    """grad_y rows for slots [slot_lo, slot_hi) (all slots by default): grad_out is
    [n_tok, H] float32 or bf16 bits; slots holding no entry keep `fill`."""
    lib = _load()
    grad_out = np.ascontiguousarray(grad_out)
    assert grad_out.dtype == _row_type(gout_dtype)
    dst = np.ascontiguousarray(dst, dtype=np.int32).reshape(-1)
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    H = grad_out.shape[-1]
    if slot_hi is None:
        slot_hi = dst.size
    out = np.full((slot_hi - slot_lo, H), fill, dtype=_row_type(y_dtype))
    lib.oracle_combine_backward_y(dst.size, K, H, gout_dtype, y_dtype, _ptr(grad_out), _ptr(w),
                                  _ptr(dst), slot_lo, slot_hi, _ptr(out))
    return out


def combine_backward_w(dst: np.ndarray, K: int, grad_out: np.ndarray, y_rows: np.ndarray,
                       gout_dtype: int, y_dtype: int) -> np.ndarray:
    """grad_w [n_tok*K] in binary64; y_rows[a] is the expert-output row of entry a."""
    lib = _load()
    grad_out = np.ascontiguousarray(grad_out)
    y_rows = np.ascontiguousarray(y_rows)
    assert grad_out.dtype == _row_type(gout_dtype) and y_rows.dtype == _row_type(y_dtype)
    dst = np.ascontiguousarray(dst, dtype=np.int32).reshape(-1)
    n_tok, H = grad_out.shape
    assert dst.size == n_tok * K and y_rows.shape == (dst.size, H)
    gw = np.zeros(dst.size, dtype=np.float64)
    lib.oracle_combine_backward_w(n_tok, K, H, gout_dtype, y_dtype, _ptr(grad_out), _ptr(y_rows),
                                  _ptr(dst), _ptr(gw))
    return gw


def dispatch_backward(dst: np.ndarray, K: int, grad_recv: np.ndarray, in_dtype: int,
                      out_dtype: int) -> np.ndarray:
    """grad_hidden [n_tok, H]: grad_recv is [n_slots, H] float32 or bf16 bits."""
    lib = _load()
    grad_recv = np.ascontiguousarray(grad_recv)
    assert grad_recv.dtype == _row_type(in_dtype)
    dst = np.ascontiguousarray(dst, dtype=np.int32).reshape(-1)
    H = grad_recv.shape[-1]
    n_tok = dst.size // K
    out = np.zeros((n_tok, H), dtype=_row_type(out_dtype))
    lib.oracle_dispatch_backward(n_tok, K, H, in_dtype, out_dtype, _ptr(grad_recv), _ptr(dst),
                                 _ptr(out))
    return out
