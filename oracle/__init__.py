"""CPU oracle of the Q4_0 W4A8 MoE expert matmul -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it;
the two implementations share no code.

This module is argument marshalling over ``liboracle.so`` (``oracle.c``, plain
single-threaded C compiled with ``-O2 -fno-fast-math -ffp-contract=off``);
every step of the arithmetic is in ``oracle.c``, which cites the page passages
and lists the readings it takes (R1..R9).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_Q4_ORACLE_LIB names another build of oracle.c to load (the sanitizer run of tests/run_sanitizers.py)
_BUILT = os.path.join(_HERE, "liboracle.so")  # where build() writes
_LIB_PATH = os.environ.get("MOE_Q4_ORACLE_LIB") or _BUILT
_lib = None

FLAG_RMSNORM = 1
FLAG_ACCUMULATE = 2
FLAG_EXACT_ACT = 4


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           src, "-o", _BUILT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_BUILT + ".tmp", _BUILT)
    return _BUILT


class _Experts(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("gate_qs", ctypes.c_void_p), ("up_qs", ctypes.c_void_p), ("down_qs", ctypes.c_void_p),
                ("gate_d", ctypes.c_void_p), ("up_d", ctypes.c_void_p), ("down_d", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_q4_dequant.argtypes = [p, p, i64, i64, p]
    lib.orc_q8_quantize.argtypes = [p, i64, i64, u32, p, p]
    lib.orc_block_dots.argtypes = [p, i64, i64, p, i64, p]
    lib.orc_gemv.argtypes = [p, p, i64, i64, p, p, i64, p]
    lib.orc_route.argtypes = [p, i32, i32, i32, p, p, p, p]
    lib.orc_router_logits.argtypes = [p, i64, i64, p, i64, u32, p]
    lib.orc_round_to_half.argtypes = [ctypes.c_double]
    lib.orc_round_to_half.restype = ctypes.c_double
    lib.orc_moe_layer_a16.argtypes = [ctypes.POINTER(_Experts), p, i32, i32, p, p, p, i32, u32, p, p]
    lib.orc_moe_layer.argtypes = [ctypes.POINTER(_Experts), p, p, i32, i32, p, p, p, i32, u32, p,
                                  p, p, p, p, p, p, p, p, p]
    for f in (lib.orc_q4_dequant, lib.orc_q8_quantize, lib.orc_block_dots, lib.orc_gemv, lib.orc_route,
              lib.orc_moe_layer):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def half_to_double(h: int) -> float:
    return _load().orc_half_to_double(int(h))


def q4_dequant(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """qs [rows][K/2] uint8, d [rows][K/32] fp16 bits -> fp64 [rows][K]."""
    qs, d = _c(qs, np.uint8), _c(d, np.uint16)
    rows, K = qs.shape[0], qs.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    _check(_load().orc_q4_dequant(_p(qs), _p(d), rows, K, _p(out)), "q4_dequant")
    return out


def q8_quantize(x: np.ndarray, flags: int = 0):
    """x [rows][cols] fp32 -> (xq int8 [rows][cols], xd fp32 [rows][cols/32])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    xq = np.empty((rows, cols), np.int8)
    xd = np.empty((rows, cols // 32), np.float32)
    _check(_load().orc_q8_quantize(_p(x), rows, cols, flags, _p(xq), _p(xd)), "q8_quantize")
    return xq, xd


def block_dots(qs: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """qs [rows][K/2], xq [T][K] -> int32 [T][rows][K/32]."""
    qs, xq = _c(qs, np.uint8), _c(xq, np.int8)
    rows, K = qs.shape[0], qs.shape[1] * 2
    T = xq.shape[0]
    assert xq.shape[1] == K
    out = np.empty((T, rows, K // 32), np.int32)
    _check(_load().orc_block_dots(_p(qs), rows, K, _p(xq), T, _p(out)), "block_dots")
    return out


def gemv(qs: np.ndarray, d: np.ndarray, xq: np.ndarray, xd: np.ndarray) -> np.ndarray:
    """W4A8 matvec: qs [N][K/2], d [N][K/32], xq [T][K], xd [T][K/32] -> fp32 [T][N]."""
    qs, d, xq, xd = _c(qs, np.uint8), _c(d, np.uint16), _c(xq, np.int8), _c(xd, np.float32)
    N, K = qs.shape[0], qs.shape[1] * 2
    T = xq.shape[0]
    y = np.empty((T, N), np.float32)
    _check(_load().orc_gemv(_p(qs), _p(d), N, K, _p(xq), _p(xd), T, _p(y)), "gemv")
    return y


def route(logits: np.ndarray, k: int):
    """logits [T][E] fp32 -> (topk_ids [T][k], topk_w [T][k], expert_offsets [E+1], sorted_pairs [T*k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    off = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    _check(_load().orc_route(_p(logits), T, E, k, _p(ids), _p(w), _p(off), _p(sp)), "route")
    return ids, w, off, sp


def round_to_half(v: float) -> float:
    """The nearest fp16 value of v (ties to even), as a Python float (R11)."""
    return float(_load().orc_round_to_half(float(v)))


def moe_layer_a16(es, x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, tokens=None, flags: int = 0,
                  y: np.ndarray | None = None, want_h: bool = False):
    """One MoE layer, W4A16 (R11): x [T][H] fp32 rows.  FLAG_EXACT_ACT: the fp64 FFN with nothing rounded.
    Returns y [T][H] fp32 and, with want_h, h [P][I] fp32 in pair order (as carried to the down projection)."""
    x = _c(x, np.float32)
    ids, w = _c(topk_ids, np.int32), _c(topk_w, np.float32)
    T, k = ids.shape
    H, I = es.H, es.I
    if y is None:
        y = np.zeros((T, H), np.float32)
    else:
        assert y.dtype == np.float32 and y.flags["C_CONTIGUOUS"] and y.shape == (T, H)
    h = np.zeros((T * k, I), np.float32) if want_h else None
    tok = None if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    st = _experts_struct(es)
    rc = _load().orc_moe_layer_a16(ctypes.byref(st), _p(x), T, k, _p(ids), _p(w), _p(tok),
                                   0 if tok is None else len(tok), flags, _p(y), _p(h))
    _check(rc, "moe_layer_a16")
    return (y, h) if want_h else y


def router_logits(x: np.ndarray, wr: np.ndarray, flags: int = 0) -> np.ndarray:
    """x [T][H] fp32, router weights wr [E][H] fp32 -> logits [T][E] fp32 (R10; R8 with FLAG_RMSNORM)."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == H
    out = np.empty((T, E), np.float32)
    _check(_load().orc_router_logits(_p(x), T, H, _p(wr), E, flags, _p(out)), "router_logits")
    return out


def _experts_struct(es) -> _Experts:
    arrs = [np.ascontiguousarray(a) for a in (es.gate_qs, es.up_qs, es.down_qs, es.gate_d, es.up_d, es.down_d)]
    s = _Experts(es.E, es.H, es.I, *[a.ctypes.data for a in arrs])
    s._keep = arrs  # keep buffers alive
    return s


def new_intermediates(P: int, I: int) -> dict:
    """Zeroed output arrays for moe_layer's intermediates (pair order): g, u, h [P][I] fp32, hq [P][I] int8,
    hd [P][I/32] fp32, and sg, su [P][I] fp64 (sum over blocks of |d_w d_a isum| of each gate / up output)."""
    return dict(g=np.zeros((P, I), np.float32), u=np.zeros((P, I), np.float32), h=np.zeros((P, I), np.float32),
                hq=np.zeros((P, I), np.int8), hd=np.zeros((P, I // 32), np.float32),
                sg=np.zeros((P, I), np.float64), su=np.zeros((P, I), np.float64))


def moe_layer(es, xq: np.ndarray, xd: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray,
              tokens=None, flags: int = 0, y: np.ndarray | None = None, want_intermediates: bool = False,
              hq_in: np.ndarray | None = None, hd_in: np.ndarray | None = None, inter: dict | None = None):
    """One MoE layer on Q8_0 activations.

    Returns y [T][H] fp32 (a new array, or ``y`` updated in place) and, with
    ``want_intermediates`` (or a preallocated ``inter`` from
    new_intermediates, filled in place: rows of other tokens are untouched, so
    calls on disjoint token sets may share it from several threads), a dict of
    g, u, h [P][I] fp32, hq [P][I] int8, hd [P][I/32] fp32 and sg, su [P][I]
    fp64 indexed by pair id p = t*k + j (rows of tokens not computed are left
    as they were).  ``hq_in``/``hd_in`` ([P][I], [P][I/32], pair order)
    replace the oracle's own re-quantised h in the down projection.  The C
    call releases the GIL.
    """
    xq, xd = _c(xq, np.int8), _c(xd, np.float32)
    ids, w = _c(topk_ids, np.int32), _c(topk_w, np.float32)
    T, k = ids.shape
    H, I = es.H, es.I
    P = T * k
    if y is None:
        y = np.zeros((T, H), np.float32)
    else:
        assert y.dtype == np.float32 and y.flags["C_CONTIGUOUS"] and y.shape == (T, H)
    tok = None if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    if inter is not None:
        want_intermediates = True
        for name, dt, cols in (("g", np.float32, I), ("u", np.float32, I), ("h", np.float32, I),
                               ("hq", np.int8, I), ("hd", np.float32, I // 32), ("sg", np.float64, I),
                               ("su", np.float64, I)):
            a = inter[name]
            assert a.dtype == dt and a.flags["C_CONTIGUOUS"] and a.shape == (P, cols), name
    elif want_intermediates:
        inter = new_intermediates(P, I)
    else:
        inter = {}
    if hq_in is not None:
        hq_in, hd_in = _c(hq_in, np.int8), _c(hd_in, np.float32)
    st = _experts_struct(es)
    rc = _load().orc_moe_layer(ctypes.byref(st), _p(xq), _p(xd), T, k, _p(ids), _p(w), _p(tok),
                               0 if tok is None else len(tok), flags, _p(y),
                               _p(inter.get("g")), _p(inter.get("u")), _p(inter.get("h")),
                               _p(inter.get("hq")), _p(inter.get("hd")), _p(hq_in), _p(hd_in),
                               _p(inter.get("sg")), _p(inter.get("su")))
    _check(rc, "moe_layer")
    return (y, inter) if want_intermediates else y
