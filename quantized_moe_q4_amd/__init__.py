"""Python binding of libmoe_q4.so -- the MI355X Q4_0 W4A8 MoE expert matmul.

Argument marshalling only: every function checks tensor placement, dtype,
shape and contiguity, then passes raw device pointers and the current HIP
stream to the C ABI of the same name (``include/moe_q4.h``).  All arithmetic
runs in the library's HIP kernels; PyTorch only owns device memory and the
stream.  There is no fallback: without the built library every call raises.

Functions (C name in brackets):
  quantize_act  [moe_q4_quantize_act]   fp32 rows -> Q8_0 (int8 codes, fp32 block scales)
  route         [moe_q4_route]          logits -> top-k ids/weights, expert offsets, sorted pairs
  decode        [moe_q4_decode]         one MoE layer, W4A8 GEMV path (T <= 64)
  decode_static [moe_q4_decode_static]  the same with the library's static device scratch (no workspace)
  decode_fused  [moe_q4_decode_fused]   quantize + route + decode in one launch (T <= 8)
  prefill       [moe_q4_prefill]        one MoE layer, int8-MFMA grouped GEMM path
  gemv          [moe_q4_gemv]           one Q4_0 matrix times Q8_0 rows
  workspace_size, status_string, debug_block_dots, debug_prefill_dots
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_Q4_LIB names another build of the library to load (the sanitizer run of tests/run_sanitizers.py)
LIB_PATH = os.environ.get("MOE_Q4_LIB") or os.path.join(_HERE, "libmoe_q4.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_WORKSPACE = -2
ERR_UNSUPPORTED = -3
ERR_HIP = -4

QUANT_RMSNORM = 1
ACCUMULATE = 2

MAX_DECODE_TOKENS = 64
MAX_FUSED_TOKENS = 8
MAX_FUSED_HQ_BYTES = 65536
MAX_STACK_LAYERS = 48
WS_CTL_BYTES = 20480  # sync area at the start of a workspace (moe_q4_decode_fused)
WS_ERROR_OFFSET = 2112  # sticky error word among them

_lib = None


class MoeQ4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


class _CExperts(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("gate_qs", ctypes.c_void_p), ("up_qs", ctypes.c_void_p), ("down_qs", ctypes.c_void_p),
                ("gate_d", ctypes.c_void_p), ("up_d", ctypes.c_void_p), ("down_d", ctypes.c_void_p)]


EXPORTED = ("moe_q4_quantize_act", "moe_q4_route", "moe_q4_workspace_size", "moe_q4_decode", "moe_q4_decode_fused",
            "moe_q4_prefill", "moe_q4_gemv", "moe_q4_debug_block_dots", "moe_q4_debug_prefill_dots",
            "moe_q4_router_logits", "moe_q4_prefill_a16", "moe_q4_prefill_a16_workspace_size", "moe_q4_probe_read", "moe_q4_probe_mfma_i8", "moe_q4_probe_w4a8_step", "moe_q4_decode_stack",
            "moe_q4_stack_workspace_size", "moe_q4_status_string", "moe_q4_decode_static",
            "moe_q4_decode_stack_batch", "moe_q4_stack_batch_workspace_size")


def load_library(path: str = LIB_PATH):
    """Load libmoe_q4.so and declare its signatures (no device work)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m quantized_moe_q4_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    p, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    pe = ctypes.POINTER(_CExperts)
    sig = {
        "moe_q4_quantize_act": [p, i64, i64, u32, p, p, p],
        "moe_q4_route": [p, i32, i32, i32, p, p, p, p, p],
        "moe_q4_workspace_size": [i32, i32, i32, i32, i32],
        "moe_q4_decode": [pe, p, p, i32, i32, p, p, p, p, u32, p, p, sz, p],
        "moe_q4_decode_static": [pe, p, p, i32, i32, p, p, p, p, u32, p, p],
        "moe_q4_decode_fused": [pe, p, p, i32, i32, u32, p, p, p, p, p, p, sz, p],
        "moe_q4_prefill": [pe, p, p, i32, i32, p, p, p, p, u32, p, p, sz, p],
        "moe_q4_gemv": [p, p, i32, i32, p, p, i32, p, p],
        "moe_q4_debug_block_dots": [p, i32, i32, p, i32, i32, p, p],
        "moe_q4_debug_prefill_dots": [pe, p, p, i32, i32, p, p, i32, p, p, sz, p],
        "moe_q4_router_logits": [p, i32, i32, p, i32, u32, p, p],
        "moe_q4_prefill_a16": [pe, p, i32, i32, p, p, p, p, u32, p, p, sz, p],
        "moe_q4_prefill_a16_workspace_size": [i32, i32, i32, i32],
        "moe_q4_probe_read": [p, sz, p, p],
        "moe_q4_probe_mfma_i8": [i32, i32, p, p],
        "moe_q4_probe_w4a8_step": [i32, i32, p, p],
        "moe_q4_decode_stack": [pe, i32, p, i32, u32, p, p, p, p, p, sz, p],
        "moe_q4_stack_workspace_size": [i32],
        "moe_q4_decode_stack_batch": [pe, i32, i32, p, i32, u32, p, p, p, p, p, sz, p],
        "moe_q4_stack_batch_workspace_size": [i32, i32, i32, i32, i32, i32],
        "moe_q4_status_string": [ctypes.c_int],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.moe_q4_workspace_size.restype = sz
    lib.moe_q4_prefill_a16_workspace_size.restype = sz
    lib.moe_q4_stack_workspace_size.restype = sz
    lib.moe_q4_stack_batch_workspace_size.restype = sz
    lib.moe_q4_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().moe_q4_status_string(int(status)).decode()


def workspace_size(T: int, E: int, k: int, H: int, I: int) -> int:
    return int(load_library().moe_q4_workspace_size(T, E, k, H, I))


def new_workspace(T: int, E: int, k: int, H: int, I: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (its sync words must start at zero for decode_fused)."""
    return torch.zeros(max(workspace_size(T, E, k, H, I), WS_CTL_BYTES), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ helpers
def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _call(fn: str, *args):
    rc = getattr(load_library(), fn)(*args)
    if rc != OK:
        raise MoeQ4Error(fn, rc)


@dataclass
class Experts:
    """One layer's experts on the device (structure of arrays, see moe_q4.h)."""
    gate_qs: torch.Tensor  # uint8 [E][I][H/2]
    up_qs: torch.Tensor    # uint8 [E][I][H/2]
    down_qs: torch.Tensor  # uint8 [E][H][I/2]
    gate_d: torch.Tensor   # int16 (fp16 bits) [E][I][H/32]
    up_d: torch.Tensor
    down_d: torch.Tensor

    @property
    def E(self) -> int:
        return self.gate_qs.shape[0]

    @property
    def I(self) -> int:
        return self.gate_qs.shape[1]

    @property
    def H(self) -> int:
        return self.gate_qs.shape[2] * 2

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.gate_qs, self.up_qs, self.down_qs, self.gate_d, self.up_d, self.down_d))

    def expert_bytes(self) -> int:
        return self.nbytes // self.E

    def _c(self) -> _CExperts:
        E, H, I = self.E, self.H, self.I
        ptrs = [
            _dev(self.gate_qs, "gate_qs", torch.uint8, (E, I, H // 2)),
            _dev(self.up_qs, "up_qs", torch.uint8, (E, I, H // 2)),
            _dev(self.down_qs, "down_qs", torch.uint8, (E, H, I // 2)),
            _dev(self.gate_d, "gate_d", torch.int16, (E, I, H // 32)),
            _dev(self.up_d, "up_d", torch.int16, (E, I, H // 32)),
            _dev(self.down_d, "down_d", torch.int16, (E, H, I // 32)),
        ]
        return _CExperts(E, H, I, *ptrs)


# ------------------------------------------------------------------ API
def quantize_act(x: torch.Tensor, flags: int = 0, xq: torch.Tensor | None = None, xd: torch.Tensor | None = None,
                 stream=None):
    """x [rows][cols] fp32 -> (xq int8 [rows][cols], xd fp32 [rows][cols/32])."""
    rows, cols = x.shape
    if xq is None:
        xq = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if xd is None:
        xd = torch.empty((rows, cols // 32), dtype=torch.float32, device=x.device)
    _call("moe_q4_quantize_act", _dev(x, "x", torch.float32), rows, cols, flags,
          _dev(xq, "xq", torch.int8, (rows, cols)), _dev(xd, "xd", torch.float32, (rows, cols // 32)),
          _stream(stream))
    return xq, xd


def route(logits: torch.Tensor, k: int, out=None, stream=None):
    """logits [T][E] fp32 -> (topk_ids [T][k] int32, topk_w [T][k] fp32, expert_offsets [E+1], sorted_pairs [T*k])."""
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev))
    ids, w, off, sp = out
    _call("moe_q4_route", _dev(logits, "logits", torch.float32), T, E, k, _dev(ids, "topk_ids", torch.int32, (T, k)),
          _dev(w, "topk_w", torch.float32, (T, k)), _dev(off, "expert_offsets", torch.int32, (E + 1,)),
          _dev(sp, "sorted_pairs", torch.int32, (T * k,)), _stream(stream))
    return ids, w, off, sp


def _layer(fn: str, experts: Experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y, ws,
           stream):
    T, k = topk_ids.shape
    E, H, I = experts.E, experts.H, experts.I
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=xq.device)
    if ws is None:
        ws = new_workspace(T, E, k, H, I, xq.device)
    c = experts._c()
    _call(fn, ctypes.byref(c), _dev(xq, "xq", torch.int8, (T, H)), _dev(xd, "xd", torch.float32, (T, H // 32)), T, k,
          _dev(topk_ids, "topk_ids", torch.int32, (T, k)), _dev(topk_w, "topk_w", torch.float32, (T, k)),
          _dev(expert_offsets, "expert_offsets", torch.int32, (E + 1,)),
          _dev(sorted_pairs, "sorted_pairs", torch.int32, (T * k,)), flags, _dev(y, "y", torch.float32, (T, H)),
          _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return y, ws


def decode(experts: Experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags: int = 0, y=None,
           ws=None, stream=None):
    """One MoE layer on the W4A8 GEMV path; returns (y [T][H], ws)."""
    return _layer("moe_q4_decode", experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y, ws,
                  stream)


STATIC_SCRATCH_BYTES = 8 << 20


def decode_static(experts: Experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags: int = 0, y=None,
                  stream=None):
    """moe_q4_decode without a workspace: the library's static per-GPU device scratch (8 MiB) stands in for it,
    so the call allocates nothing (y must be given for that).  Calls that overlap on one GPU race.  Returns y."""
    T, k = topk_ids.shape
    E, H = experts.E, experts.H
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=xq.device)
    c = experts._c()
    _call("moe_q4_decode_static", ctypes.byref(c), _dev(xq, "xq", torch.int8, (T, H)),
          _dev(xd, "xd", torch.float32, (T, H // 32)), T, k, _dev(topk_ids, "topk_ids", torch.int32, (T, k)),
          _dev(topk_w, "topk_w", torch.float32, (T, k)), _dev(expert_offsets, "expert_offsets", torch.int32, (E + 1,)),
          _dev(sorted_pairs, "sorted_pairs", torch.int32, (T * k,)), flags, _dev(y, "y", torch.float32, (T, H)),
          _stream(stream))
    return y


def decode_fused(experts: Experts, x: torch.Tensor, logits: torch.Tensor, k: int, flags: int = 0, out=None, y=None,
                 ws=None, stream=None):
    """Quantize + route + one MoE decode layer in one launch (T <= 8).

    x [T][H] fp32, logits [T][E] fp32; flags: QUANT_RMSNORM and/or ACCUMULATE.
    Returns (y [T][H], (topk_ids, topk_w, expert_offsets, sorted_pairs), ws).  y may be x (in place).
    ws must be a zero-filled workspace (new_workspace) or one only ever used by this library.
    """
    T, H = x.shape
    E = experts.E
    dev = x.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev))
    ids, w, off, sp = out
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
    if ws is None:
        ws = new_workspace(T, E, k, H, experts.I, dev)
    c = experts._c()
    _call("moe_q4_decode_fused", ctypes.byref(c), _dev(x, "x", torch.float32, (T, experts.H)),
          _dev(logits, "logits", torch.float32, (T, E)), T, k, flags, _dev(ids, "topk_ids", torch.int32, (T, k)),
          _dev(w, "topk_w", torch.float32, (T, k)), _dev(off, "expert_offsets", torch.int32, (E + 1,)),
          _dev(sp, "sorted_pairs", torch.int32, (T * k,)), _dev(y, "y", torch.float32, (T, experts.H)),
          _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return y, out, ws


def stack_workspace_size(H: int) -> int:
    return int(load_library().moe_q4_stack_workspace_size(H))


def new_stack_workspace(H: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for decode_stack (it may also serve decode_fused calls on the same stream)."""
    return torch.zeros(stack_workspace_size(H), dtype=torch.uint8, device=device)


class StackLayers:
    """The expert sets of a layer stack, checked and packed once for repeated decode_stack calls."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.L = len(self.layers)
        self.E, self.H, self.I = self.layers[0].E, self.layers[0].H, self.layers[0].I
        self.c = (_CExperts * self.L)(*[ex._c() for ex in self.layers])


def decode_stack(layers, h: torch.Tensor, logits: torch.Tensor, k: int, flags: int = 0, h_all=None,
                 hq_all=None, hd_all=None, ws=None, stream=None):
    """L MoE decode layers of one token in one launch (moe_q4_decode_stack).

    layers: list of L Experts (same E, H, I) or a StackLayers; h [H] or [1][H] fp32, updated in place
    (h_0 in, h_L out); logits [L][E] or [L][1][E] fp32; flags: QUANT_RMSNORM and/or ACCUMULATE at every
    layer.  Optional outputs: h_all [L][H] fp32; hq_all [L][k][I] int8 with hd_all [L][k][I/32] fp32.
    Returns (h, ws).
    """
    st = layers if isinstance(layers, StackLayers) else StackLayers(layers)
    L, E, H, I = st.L, st.E, st.H, st.I
    if h.numel() != H or logits.numel() != L * E:
        raise ValueError("decode_stack: h must hold H values and logits L * E")
    if ws is None:
        ws = new_stack_workspace(H, h.device)
    arr = st.c
    opt = lambda t, name, dtype, shape: 0 if t is None else _dev(t, name, dtype, shape)
    _call("moe_q4_decode_stack", arr, L, _dev(logits, "logits", torch.float32, logits.shape), k, flags,
          _dev(h, "h", torch.float32, h.shape), opt(h_all, "h_all", torch.float32, (L, H)),
          opt(hq_all, "hq_all", torch.int8, (L, k, I)), opt(hd_all, "hd_all", torch.float32, (L, k, I // 32)),
          _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return h, ws


def stack_batch_workspace_size(L: int, T: int, E: int, k: int, H: int, I: int) -> int:
    return int(load_library().moe_q4_stack_batch_workspace_size(L, T, E, k, H, I))


def new_stack_batch_workspace(L: int, T: int, E: int, k: int, H: int, I: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for decode_stack_batch."""
    n = stack_batch_workspace_size(L, T, E, k, H, I)
    if n == 0:
        raise ValueError("decode_stack_batch: shape not supported")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def decode_stack_batch(layers, h: torch.Tensor, logits: torch.Tensor, k: int, flags: int = 0, h_all=None,
                       hq_all=None, hd_all=None, ws=None, stream=None):
    """L MoE decode layers of T <= 16 tokens in one persistent launch (moe_q4_decode_stack_batch).

    layers: list of L Experts or a StackLayers; h [T][H] fp32 updated in place (h_0 in, h_L out);
    logits [L][T][E] fp32; flags: QUANT_RMSNORM and/or ACCUMULATE at every layer.  Optional outputs:
    h_all [L][T][H]; hq_all [L][T*k][I] int8 with hd_all [L][T*k][I/32] fp32 (sorted-pair order).
    Returns (h, ws).
    """
    st = layers if isinstance(layers, StackLayers) else StackLayers(layers)
    L, E, H, I = st.L, st.E, st.H, st.I
    T = h.shape[0]
    if h.shape != (T, H) or logits.numel() != L * T * E:
        raise ValueError("decode_stack_batch: h must be [T][H] and logits [L][T][E]")
    if ws is None:
        ws = new_stack_batch_workspace(L, T, E, k, H, I, h.device)
    opt = lambda t, name, dtype, shape: 0 if t is None else _dev(t, name, dtype, shape)
    P = T * k
    _call("moe_q4_decode_stack_batch", st.c, L, T, _dev(logits, "logits", torch.float32, logits.shape), k, flags,
          _dev(h, "h", torch.float32, (T, H)), opt(h_all, "h_all", torch.float32, (L, T, H)),
          opt(hq_all, "hq_all", torch.int8, (L, P, I)), opt(hd_all, "hd_all", torch.float32, (L, P, I // 32)),
          _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return h, ws


def workspace_error(ws: torch.Tensor) -> int:
    """The sticky error word of a workspace's sync area (nonzero: a fused call's bounded wait gave up)."""
    return int(ws[WS_ERROR_OFFSET:WS_ERROR_OFFSET + 4].view(torch.int32).item())


def prefill(experts: Experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags: int = 0, y=None,
            ws=None, stream=None):
    """One MoE layer on the grouped int8-MFMA GEMM path; returns (y [T][H], ws)."""
    return _layer("moe_q4_prefill", experts, xq, xd, topk_ids, topk_w, expert_offsets, sorted_pairs, flags, y, ws,
                  stream)


def workspace_views(ws: torch.Tensor, T: int, k: int, I: int):
    """(hq int8 [P][I], hd fp32 [P][I/32]) views of a decode/prefill workspace, rows in sorted-pair order."""
    P = T * k
    base = WS_CTL_BYTES
    off = base + (P * I + 255) // 256 * 256
    hq = ws[base:base + P * I].view(torch.int8).view(P, I)
    hd = ws[off:off + P * (I // 32) * 4].view(torch.float32).view(P, I // 32)
    return hq, hd


def gemv(qs: torch.Tensor, d: torch.Tensor, xq: torch.Tensor, xd: torch.Tensor, y=None, stream=None):
    """One Q4_0 matrix qs [N][K/2], d [N][K/32] (int16 fp16 bits) times Q8_0 rows xq [T][K] -> y [T][N]."""
    N, K = qs.shape[0], qs.shape[1] * 2
    T = xq.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=qs.device)
    _call("moe_q4_gemv", _dev(qs, "qs", torch.uint8, (N, K // 2)), _dev(d, "d", torch.int16, (N, K // 32)), N, K,
          _dev(xq, "xq", torch.int8, (T, K)), _dev(xd, "xd", torch.float32, (T, K // 32)), T,
          _dev(y, "y", torch.float32, (T, N)), _stream(stream))
    return y


def prefill_a16_workspace_size(T: int, k: int, H: int, I: int) -> int:
    return int(load_library().moe_q4_prefill_a16_workspace_size(T, k, H, I))


def prefill_a16(experts: Experts, x, topk_ids, topk_w, expert_offsets, sorted_pairs, flags: int = 0, y=None,
                ws=None, stream=None):
    """W4A16 prefill layer: x [T][H] fp32 and the routing -> (y [T][H] fp32, ws).  ws holds x and h in fp16."""
    T = x.shape[0]
    k = topk_ids.shape[1] if T > 0 else int(topk_ids.shape[-1])
    E, H, I = experts.E, experts.H, experts.I
    if y is None:
        y = torch.zeros((T, H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(prefill_a16_workspace_size(T, k, H, I), 256), dtype=torch.uint8, device=x.device)
    c = experts._c()
    _call("moe_q4_prefill_a16", ctypes.byref(c), _dev(x, "x", torch.float32, (T, H)), T, k,
          _dev(topk_ids, "topk_ids", torch.int32, (T, k)), _dev(topk_w, "topk_w", torch.float32, (T, k)),
          _dev(expert_offsets, "expert_offsets", torch.int32, (E + 1,)),
          _dev(sorted_pairs, "sorted_pairs", torch.int32, (T * k,)), flags, _dev(y, "y", torch.float32, (T, H)),
          ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    return y, ws


def a16_views(ws: torch.Tensor, T: int, k: int, H: int, I: int):
    """(x16 [T][H], h16 [P][I]) fp16 views of a W4A16 workspace, in natural element order."""
    a = lambda v: (v + 255) // 256 * 256
    x16 = ws[:T * H * 2].view(torch.float16).view(T, H)
    h16 = ws[a(T * H * 2):a(T * H * 2) + T * k * I * 2].view(torch.float16).view(T * k, I)
    perm = torch.tensor([0, 2, 1, 3, 4, 6, 5, 7], device=ws.device)  # stored position of element j
    unperm = lambda t: t.view(t.shape[0], -1, 8)[:, :, perm].reshape(t.shape)
    return unperm(x16), unperm(h16)


def router_logits(x: torch.Tensor, wr: torch.Tensor, flags: int = 0, out=None, stream=None) -> torch.Tensor:
    """Router projection: x [T][H] fp32, router weights wr [E][H] fp32 -> logits [T][E] fp32."""
    T, H = x.shape
    E = wr.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _call("moe_q4_router_logits", _dev(x, "x", torch.float32, (T, H)), T, H, _dev(wr, "wr", torch.float32, (E, H)), E,
          flags, _dev(out, "logits", torch.float32, (T, E)), _stream(stream))
    return out


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """Stream-read every byte of a contiguous device tensor once; returns the bytes read."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: must be a contiguous device tensor")
    _call("moe_q4_probe_read", buf.data_ptr(), nbytes, _dev(sink, "sink", torch.int32), _stream(stream))
    return nbytes


def probe_mfma_i8(iters: int, workgroups: int, sink: torch.Tensor, stream=None) -> int:
    """Back-to-back int8 32x32x32 MFMA on registers; returns the int ops issued."""
    _call("moe_q4_probe_mfma_i8", int(iters), int(workgroups), _dev(sink, "sink", torch.int32), _stream(stream))
    return 262144 * int(iters) * 4 * int(workgroups)


def probe_w4a8_step(iters: int, workgroups: int, sink: torch.Tensor, stream=None) -> int:
    """The W4A8 prefill step (2 int8 MFMA + 2 scale FMAs per output) on registers; returns the int ops issued."""
    _call("moe_q4_probe_w4a8_step", int(iters), int(workgroups), _dev(sink, "sink", torch.float32), _stream(stream))
    return 131072 * int(iters) * 4 * int(workgroups)


def debug_block_dots(qs: torch.Tensor, xq: torch.Tensor, down_walk: bool = False, stream=None):
    """Exact int32 block dots through the decode row walk: -> int32 [T][N][K/32]."""
    N, K = qs.shape[0], qs.shape[1] * 2
    T = xq.shape[0]
    out = torch.empty((T, N, K // 32), dtype=torch.int32, device=qs.device)
    _call("moe_q4_debug_block_dots", _dev(qs, "qs", torch.uint8, (N, K // 2)), N, K, _dev(xq, "xq", torch.int8, (T, K)),
          T, int(bool(down_walk)), _dev(out, "out", torch.int32), _stream(stream))
    return out


def debug_prefill_dots(experts: Experts, xq, xd, expert_offsets, sorted_pairs, k: int, which: int, ws,
                       stream=None):
    """Exact int32 block dots through the prefill MFMA kernels (which=0 gate/up, 1 down), rows in sorted order."""
    T = xq.shape[0]
    E, H, I = experts.E, experts.H, experts.I
    P = T * k
    shape = (P, 2, I, H // 32) if which == 0 else (P, H, I // 32)
    out = torch.empty(shape, dtype=torch.int32, device=xq.device)
    c = experts._c()
    _call("moe_q4_debug_prefill_dots", ctypes.byref(c), _dev(xq, "xq", torch.int8, (T, H)),
          _dev(xd, "xd", torch.float32, (T, H // 32)), T, k, _dev(expert_offsets, "expert_offsets", torch.int32),
          _dev(sorted_pairs, "sorted_pairs", torch.int32), which, _dev(out, "out", torch.int32),
          _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream))
    return out
