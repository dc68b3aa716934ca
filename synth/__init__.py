"""Seeded synthetic inputs shared by the oracle, the tests and the bench.

This package draws bytes and numbers; it holds no arithmetic of the quantized
MoE method.  Every tensor is a pure function of (seed, tensor id, element
index) through a counter-based SplitMix64 stream (``synth.c`` states the exact
definition), so any slice can be regenerated independently.

Workloads (the five synthetic cases the library is measured and tested on):

====  ===========================================================================
 0    one Q4_0 matrix N=512 x K=2048 and one activation vector x ~ N(0,1)
 1    one MoE layer, decode, T=1: hidden 2048, 128 experts (gate/up 512x2048,
      down 2048x512), logits ~ N(0,1), top-8
 2    one MoE layer, prefill, T=947 tokens, 128 experts, top-8
 3    skewed prefill, T=4096, 256 experts, top-8, logits ~ N(0,1) plus the bias
      2*log(Zipf(1.1) weight of expert e) = -2.2*log(e+1)
 4    40-layer stack, 128 experts per layer, decode batches 1, 4 and 16, fresh
      N(0,1) logits per layer
====  ===========================================================================

Weight distributions: nibbles uniform on 0..15, fp16 scales uniform on
[0.002, 0.02] rounded to nearest-even fp16.  The seed of workload i is i + 1.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_Q4_SYNTH_LIB names another build of synth.c to load (the sanitizer run of tests/run_sanitizers.py)
_BUILT = os.path.join(_HERE, "libsynth.so")  # where build() writes
_LIB_PATH = os.environ.get("MOE_Q4_SYNTH_LIB") or _BUILT
_lib = None

SCALE_LO = 0.002
SCALE_HI = 0.02
ZIPF_S = 1.1

# tensor-id space
TID_X = 1
TID_LOGITS = 2
TID_ROUTER = 3
MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2
ROLE_QS, ROLE_D = 0, 1


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP, no FMA contraction)."""
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           src, "-o", _BUILT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_BUILT + ".tmp", _BUILT)
    return _BUILT


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    lib.synth_u64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_uniform_f64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, p]
    lib.synth_biased_logits_f32.argtypes = [u64, u64, i64, i64, ctypes.c_double, p]
    lib.synth_nibble_bytes.argtypes = [u64, u64, u64, i64, p]
    lib.synth_scales_f16.argtypes = [u64, u64, u64, i64, ctypes.c_double, ctypes.c_double, p]
    for f in (lib.synth_u64, lib.synth_uniform_f64, lib.synth_normal_f32, lib.synth_biased_logits_f32,
              lib.synth_nibble_bytes, lib.synth_scales_f16):
        f.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- raw streams
def u64(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_u64(seed, tid, start, n, _ptr(out))
    return out


def uniform(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform_f64(seed, tid, start, n, _ptr(out))
    return out


def normal(seed: int, tid: int, shape, start: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, tid, start, n, _ptr(out))
    return out


def biased_logits(seed: int, tid: int, T: int, E: int, s_bias: float) -> np.ndarray:
    out = np.empty((T, E), np.float32)
    _load().synth_biased_logits_f32(seed, tid, T, E, s_bias, _ptr(out))
    return out


def nibble_bytes(seed: int, tid: int, nbytes: int, start: int = 0, out: np.ndarray | None = None):
    if out is None:
        out = np.empty(nbytes, np.uint8)
    _load().synth_nibble_bytes(seed, tid, start, nbytes, _ptr(out))
    return out


def scales_f16(seed: int, tid: int, n: int, start: int = 0, out: np.ndarray | None = None):
    if out is None:
        out = np.empty(n, np.uint16)
    _load().synth_scales_f16(seed, tid, start, n, SCALE_LO, SCALE_HI, _ptr(out))
    return out


# ------------------------------------------------------------ tensor ids
def expert_tid(layer: int, expert: int, mat: int, role: int) -> int:
    return (1 << 40) | (layer << 24) | (expert << 8) | (mat << 2) | role


def x_tid(T: int) -> int:
    return TID_X | (T << 16)


def logits_tid(layer: int, T: int) -> int:
    return TID_LOGITS | (layer << 8) | (T << 32)


def router_tid(layer: int, E: int, H: int) -> int:
    return TID_ROUTER | (layer << 8) | (E << 20) | (H << 40)


def router_weights(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    """Router projection [E][H] fp32: N(0, 1) / sqrt(H), so that logits of N(0, 1) rows are about N(0, 1)."""
    return (normal(seed, router_tid(layer, E, H), (E, H)) * np.float32(1.0 / math.sqrt(H))).astype(np.float32)


# ------------------------------------------------------------ Q4_0 matrices
def q4_matrix(seed: int, layer: int, expert: int, mat: int, rows: int, cols: int,
              qs_out: np.ndarray | None = None, d_out: np.ndarray | None = None):
    """One Q4_0 matrix [rows][cols]: qs uint8 [rows][cols/2], d fp16 bits [rows][cols/32]."""
    assert cols % 32 == 0
    qs = nibble_bytes(seed, expert_tid(layer, expert, mat, ROLE_QS), rows * cols // 2,
                      out=None if qs_out is None else qs_out.reshape(-1))
    d = scales_f16(seed, expert_tid(layer, expert, mat, ROLE_D), rows * cols // 32,
                   out=None if d_out is None else d_out.reshape(-1))
    return qs.reshape(rows, cols // 2), d.reshape(rows, cols // 32)


@dataclass
class ExpertSet:
    """All experts of one layer in the library's structure-of-arrays layout."""
    E: int
    H: int
    I: int
    gate_qs: np.ndarray  # [E][I][H/2]
    up_qs: np.ndarray    # [E][I][H/2]
    down_qs: np.ndarray  # [E][H][I/2]
    gate_d: np.ndarray   # [E][I][H/32] fp16 bits
    up_d: np.ndarray     # [E][I][H/32]
    down_d: np.ndarray   # [E][H][I/32]

    @property
    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.gate_qs, self.up_qs, self.down_qs,
                                      self.gate_d, self.up_d, self.down_d))


def expert_set(seed: int, layer: int, E: int, H: int, I: int) -> ExpertSet:
    es = ExpertSet(E, H, I,
                   np.empty((E, I, H // 2), np.uint8), np.empty((E, I, H // 2), np.uint8),
                   np.empty((E, H, I // 2), np.uint8),
                   np.empty((E, I, H // 32), np.uint16), np.empty((E, I, H // 32), np.uint16),
                   np.empty((E, H, I // 32), np.uint16))
    for e in range(E):
        q4_matrix(seed, layer, e, MAT_GATE, I, H, es.gate_qs[e], es.gate_d[e])
        q4_matrix(seed, layer, e, MAT_UP, I, H, es.up_qs[e], es.up_d[e])
        q4_matrix(seed, layer, e, MAT_DOWN, H, I, es.down_qs[e], es.down_d[e])
    return es


# ------------------------------------------------------------ workloads
@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    T: int
    E: int
    k: int
    H: int = 2048
    I: int = 512
    zipf_bias: bool = False
    layers: int = 1

    @property
    def seed(self) -> int:
        return self.index + 1


WORKLOADS = {
    0: Workload(0, "gemv_512x2048", T=1, E=1, k=1),
    1: Workload(1, "moe_decode_T1_E128_k8", T=1, E=128, k=8),
    2: Workload(2, "moe_prefill_T947_E128_k8", T=947, E=128, k=8),
    3: Workload(3, "moe_prefill_skew_T4096_E256_k8", T=4096, E=256, k=8, zipf_bias=True),
    4: Workload(4, "moe_stack40_decode_E128_k8", T=16, E=128, k=8, layers=40),
}
STACK_BATCHES = (1, 4, 16)


def activations(w: Workload, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    return normal(w.seed, x_tid(T), (T, w.H))


def logits(w: Workload, layer: int = 0, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    if w.zipf_bias:
        return biased_logits(w.seed, logits_tid(layer, T), T, w.E, -2.0 * ZIPF_S)
    return normal(w.seed, logits_tid(layer, T), (T, w.E))


def gemv_matrix(w: Workload | None = None):
    """Workload 0's matrix: N=512 rows, K=2048 columns."""
    w = WORKLOADS[0] if w is None else w
    return q4_matrix(w.seed, 0, 0, MAT_GATE, 512, 2048)
