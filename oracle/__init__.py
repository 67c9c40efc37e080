"""CPU oracle of the routed MoE FFN layer (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg use this; the GPU library never does.  The
arithmetic lives in ``oracle.c`` (scalar C, double precision); this file only
marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no FMA contraction, so each product and sum rounds once)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_f16.restype = dbl
        L.oracle_f16.argtypes = [ctypes.c_uint16]
        L.oracle_bf16.restype = dbl
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_blob_layout.argtypes = [i32, i32, i32, vp]
        L.oracle_weight.restype = dbl
        L.oracle_weight.argtypes = [vp, i32, i32, i32, i32, i32, i32]
        L.oracle_dequant_matrix.argtypes = [vp, i32, i32, i32, i32, vp]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_dispatch.restype = i32
        L.oracle_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_ffn_decoded.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
        L.oracle_expert_ffn.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.oracle_combine.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.oracle_router_logits.argtypes = [vp, i32, vp, i32, i32, i32, vp]
        L.oracle_layer.restype = i32
        L.oracle_layer.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_layer_mt.restype = i32
        L.oracle_layer_mt.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def f16(bits: int) -> float:
    return float(lib().oracle_f16(bits))


def bf16(bits: int) -> float:
    return float(lib().oracle_bf16(bits))


def blob_layout(H: int, I: int, bits: int) -> list[int]:
    off = np.empty(7, np.int64)
    lib().oracle_blob_layout(H, I, bits, _p(off))
    return [int(v) for v in off]


def dequant(blob: np.ndarray, H: int, I: int, bits: int, mat: int) -> np.ndarray:
    """Decoded matrix mat (0 = Wg [I,H], 1 = Wu [I,H], 2 = Wd [H,I]) as float64."""
    blob = np.ascontiguousarray(blob, np.uint8)
    R, K = (I, H) if mat < 2 else (H, I)
    out = np.empty((R, K), np.float64)
    lib().oracle_dequant_matrix(_p(blob), H, I, bits, mat, _p(out))
    return out


def weight(blob: np.ndarray, H: int, I: int, bits: int, mat: int, r: int, c: int) -> float:
    blob = np.ascontiguousarray(blob, np.uint8)
    return float(lib().oracle_weight(_p(blob), H, I, bits, mat, r, c))


def route(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    lg = np.ascontiguousarray(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    if lib().oracle_route(_p(lg), T, E, k, _p(ids), _p(w)) != 0:
        raise ValueError("oracle_route: bad arguments")
    return ids, w


def dispatch(ids: np.ndarray, E: int) -> dict:
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    n = T * k
    offsets = np.empty(E + 1, np.int32)
    sorted_assign = np.empty(max(n, 1), np.int32)
    assign_pos = np.empty(max(n, 1), np.int32)
    active = np.empty(max(min(E, n), 1), np.int32)
    n_active = np.zeros(1, np.int32)
    if lib().oracle_dispatch(_p(ids), T, k, E, _p(offsets), _p(sorted_assign), _p(assign_pos), _p(active),
                             _p(n_active)) != 0:
        raise ValueError("oracle_dispatch: expert id out of range")
    na = int(n_active[0])
    return {"offsets": offsets, "sorted_assign": sorted_assign[:n], "assign_pos": assign_pos[:n],
            "active": active[:na], "n_active": na}


def expert_ffn(blob: np.ndarray, H: int, I: int, bits: int, x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(h [I], y [H]) of one expert on one float64 row x [H]."""
    blob = np.ascontiguousarray(blob, np.uint8)
    x = np.ascontiguousarray(x, np.float64)
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    lib().oracle_expert_ffn(_p(blob), H, I, bits, _p(x), _p(h), _p(y))
    return h, y


def ffn_decoded(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    wg, wu, wd = (np.ascontiguousarray(a, np.float64) for a in (wg, wu, wd))
    I, H = wg.shape
    x = np.ascontiguousarray(x, np.float64)
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    lib().oracle_ffn_decoded(_p(wg), _p(wu), _p(wd), H, I, _p(x), _p(h), _p(y))
    return h, y


def combine(y: np.ndarray, w: np.ndarray, residual: np.ndarray | None = None) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    T, k, H = y.shape
    r = None if residual is None else np.ascontiguousarray(residual, np.float64)
    out = np.empty((T, H), np.float64)
    lib().oracle_combine(_p(y), _p(w), T, k, H, _p(r), _p(out))
    return out


def router_logits(x: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """Router projection logits [T, E] (float64) of x (float32 values or uint16 raw bf16 bits, [T, H])
    and router weights wr_bits (uint16 raw bf16 bits, [E, H])."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        xb = 1
    elif x.dtype == np.float32:
        xb = 0
    else:
        raise TypeError("x must be float32 values or uint16 bf16 bits")
    wr = np.ascontiguousarray(wr_bits, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H)
    out = np.empty((T, E), np.float64)
    lib().oracle_router_logits(_p(x), xb, _p(wr), T, H, E, _p(out))
    return out


def default_threads() -> int:
    """Threads for oracle_layer_mt: OMP_NUM_THREADS when set, else the CPU count, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


def layer(x: np.ndarray, logits: np.ndarray, experts: np.ndarray, k: int, H: int, I: int, bits: int,
          residual: np.ndarray | None = None, want_y: bool = True, nthreads: int = 1) -> dict:
    """Whole layer.  x: float32 [T,H] values or uint16 [T,H] raw bf16 bits.
    experts: uint8 [E, stride] (expert e's blob in row e).
    nthreads > 1 runs oracle_layer_mt (same functions on the same rows, so the
    same bits); nthreads = 1 runs oracle_layer."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        xb = 1
    elif x.dtype == np.float32:
        xb = 0
    else:
        raise TypeError("x must be float32 or raw bf16 bits (uint16)")
    lg = np.ascontiguousarray(logits, np.float32)
    T, E = lg.shape
    assert x.shape == (T, H)
    experts = np.ascontiguousarray(experts, np.uint8)
    assert experts.shape[0] == E
    stride = experts.shape[1]
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    y = np.empty((T, k, H), np.float64) if want_y else None
    out = np.empty((T, H), np.float64)
    r = None if residual is None else np.ascontiguousarray(residual, np.float64)
    if nthreads > 1:
        rc = lib().oracle_layer_mt(_p(x), xb, _p(lg), _p(experts), stride, T, E, k, H, I, bits, _p(r), _p(ids),
                                   _p(w), _p(y), _p(out), int(nthreads))
    else:
        rc = lib().oracle_layer(_p(x), xb, _p(lg), _p(experts), stride, T, E, k, H, I, bits, _p(r), _p(ids), _p(w),
                                _p(y), _p(out))
    if rc != 0:
        raise ValueError("oracle_layer: bad arguments")
    return {"ids": ids, "w": w, "y": y, "out": out}
