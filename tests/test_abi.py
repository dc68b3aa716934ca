"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import quantized_moe_q4_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q4.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mq.LIB_PATH):
        from quantized_moe_q4_amd import build
        build.build()
    return mq.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_q4_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe_q4.h but not exported"
    assert sorted(mq.EXPORTED) == names


def test_status_strings(lib):
    assert mq.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert mq.status_string(code) not in ("ok", "unknown status")
    assert mq.status_string(7) == "unknown status"


def test_workspace_size(lib):
    assert mq.workspace_size(0, 128, 8, 2048, 512) == 0
    a = lambda v: (v + 255) // 256 * 256
    # 20480 bytes of sync area, then hq [P][I] int8, hd [P][I/32] fp32 and the per-pair down outputs o [P][H] fp32
    P = 947 * 8
    assert mq.workspace_size(947, 128, 8, 2048, 512) == 20480 + a(P * 512) + a(P * 16 * 4) + a(P * 2048 * 4)
    P = 16 * 8
    assert mq.workspace_size(16, 128, 8, 2048, 512) == 20480 + a(P * 512) + a(P * 16 * 4) + a(P * 2048 * 4)
    assert mq.workspace_size(1, 128, 8, 2048, 512) % 256 == 0


# Fake, aligned, never-dereferenced addresses: every call below must fail validation.
A = 1 << 20


def test_quantize_validation(lib):
    f = lib.moe_q4_quantize_act
    assert f(None, 1, 64, 0, A, A, None) == mq.ERR_INVALID_ARG
    assert f(A, 1, 48, 0, A, A, None) == mq.ERR_INVALID_ARG      # cols % 32
    assert f(A, -1, 64, 0, A, A, None) == mq.ERR_INVALID_ARG     # rows < 0
    assert f(A + 4, 1, 64, 0, A, A, None) == mq.ERR_INVALID_ARG  # x not 16-byte aligned
    assert f(A, 1, 64, 8, A, A, None) == mq.ERR_INVALID_ARG      # unknown flag
    assert f(A, 1, 32768, 0, A, A, None) == mq.ERR_UNSUPPORTED   # cols above the build's limit
    assert f(None, 0, 64, 0, None, None, None) == mq.OK          # empty input, null pointers


def test_route_validation(lib):
    f = lib.moe_q4_route
    assert f(A, 4, 8, 9, A, A, A, A, None) == mq.ERR_INVALID_ARG   # k > E
    assert f(A, 4, 8, 0, A, A, A, A, None) == mq.ERR_INVALID_ARG   # k < 1
    assert f(A, -1, 8, 2, A, A, A, A, None) == mq.ERR_INVALID_ARG  # T < 0
    assert f(None, 4, 8, 2, A, A, A, A, None) == mq.ERR_INVALID_ARG
    assert f(A, 4, 1025, 2, A, A, A, A, None) == mq.ERR_UNSUPPORTED
    assert f(A, 4, 64, 17, A, A, A, A, None) == mq.ERR_UNSUPPORTED
    assert f(None, 0, 64, 2, None, None, None, None, None) == mq.ERR_INVALID_ARG  # offsets are always written


def _experts(E=8, H=2048, I=512, ptr=A):
    return mq._CExperts(E, H, I, ptr, ptr, ptr, ptr, ptr, ptr)


@pytest.mark.parametrize("fn", ["moe_q4_decode", "moe_q4_prefill"])
def test_layer_validation(lib, fn):
    f = getattr(lib, fn)
    T, k = 4, 2
    ws_need = mq.workspace_size(T, 8, k, 2048, 512)

    def call(ex=None, T=T, k=k, flags=0, ws=A, ws_bytes=ws_need, xq=A):
        ex = _experts() if ex is None else ex
        return f(ctypes.byref(ex), xq, A, T, k, A, A, A, A, flags, A, ws, ws_bytes, None)

    assert f(None, A, A, T, k, A, A, A, A, 0, A, A, ws_need, None) == mq.ERR_INVALID_ARG
    assert call(ex=_experts(E=8, H=2040)) == mq.ERR_INVALID_ARG            # H % 32
    assert call(ex=_experts(E=8, H=4096)) == mq.ERR_UNSUPPORTED            # H outside the build
    assert call(ex=_experts(E=8, I=384)) == mq.ERR_UNSUPPORTED
    assert call(ex=_experts(E=2000)) == mq.ERR_UNSUPPORTED
    assert call(ex=_experts(ptr=A + 8)) == mq.ERR_INVALID_ARG              # weights not 16-byte aligned
    assert call(k=9) == mq.ERR_INVALID_ARG                                 # k > E
    assert call(flags=1) == mq.ERR_INVALID_ARG                             # RMSNORM is a quantize flag
    assert call(ws=None) == mq.ERR_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == mq.ERR_WORKSPACE
    assert call(ws=A + 64) == mq.ERR_WORKSPACE                             # ws not 256-byte aligned
    assert call(xq=A + 1) == mq.ERR_INVALID_ARG
    assert f(ctypes.byref(_experts()), A, A, T, k, A, A, A, A, 0, A + 4, A, ws_need, None) == mq.ERR_INVALID_ARG  # y
    if fn == "moe_q4_decode":
        need = mq.workspace_size(65, 8, k, 2048, 512)
        assert call(T=65, ws_bytes=need) == mq.ERR_UNSUPPORTED


def test_decode_static_validation(lib):
    """The static-scratch decode validates before touching the device: no HIP call on a bad argument."""
    f = lib.moe_q4_decode_static

    def call(ex=None, T=4, k=2, flags=0, xq=A, y=A):
        ex = _experts() if ex is None else ex
        return f(ctypes.byref(ex), xq, A, T, k, A, A, A, A, flags, y, None)

    assert f(None, A, A, 4, 2, A, A, A, A, 0, A, None) == mq.ERR_INVALID_ARG
    assert call(ex=_experts(E=8, H=2040)) == mq.ERR_INVALID_ARG
    assert call(ex=_experts(E=8, H=4096)) == mq.ERR_UNSUPPORTED
    assert call(k=9) == mq.ERR_INVALID_ARG
    assert call(flags=1) == mq.ERR_INVALID_ARG
    assert call(xq=A + 1) == mq.ERR_INVALID_ARG
    assert call(y=A + 4) == mq.ERR_INVALID_ARG
    assert call(T=65) == mq.ERR_UNSUPPORTED
    # beyond the 8 MiB scratch: T = 64, k = 16, H = 2048, I = 1024 needs about 9.2 MB
    assert mq.workspace_size(64, 16, 16, 2048, 1024) > mq.STATIC_SCRATCH_BYTES
    assert call(ex=_experts(E=16, I=1024), T=64, k=16) == mq.ERR_WORKSPACE
    # T == 0: a no-op, the per-token arrays may be null (and the scratch is not looked up)
    assert f(ctypes.byref(_experts()), None, None, 0, 2, None, None, None, None, 0, None, None) == mq.OK


def test_decode_fused_validation(lib):
    f = lib.moe_q4_decode_fused
    T, k = 1, 8
    ws_need = mq.workspace_size(T, 8, k, 2048, 512)

    def call(ex=None, T=T, k=k, flags=0, ws=A, ws_bytes=ws_need, x=A, logits=A, y=A):
        ex = _experts() if ex is None else ex
        return f(ctypes.byref(ex), x, logits, T, k, flags, A, A, A, A, y, ws, ws_bytes, None)

    assert call(flags=4) == mq.ERR_INVALID_ARG                             # unknown flag
    assert call(x=A + 4) == mq.ERR_INVALID_ARG                             # x not 16-byte aligned
    assert call(logits=None) == mq.ERR_INVALID_ARG
    assert call(y=A + 4) == mq.ERR_INVALID_ARG
    assert call(ws=None) == mq.ERR_WORKSPACE
    assert call(ex=_experts(E=8, H=4096)) == mq.ERR_UNSUPPORTED
    need9 = mq.workspace_size(9, 8, k, 2048, 512)
    assert call(T=9, ws_bytes=need9) == mq.ERR_UNSUPPORTED                 # above the fused token limit
    need = mq.workspace_size(8, 16, 16, 2048, 1024)                        # T*k*I = 128 KB > 64 KB
    assert call(ex=_experts(E=16, I=1024), T=8, k=16, ws_bytes=need) == mq.ERR_UNSUPPORTED
    assert f(ctypes.byref(_experts()), None, None, 0, k, 0, None, None, None, None, None, None, 0,
             None) == mq.OK                                                # T == 0: no-op


def test_decode_stack_validation(lib):
    f = lib.moe_q4_decode_stack
    need = mq.stack_workspace_size(2048)
    # sync area, h exchange, y exchange (H <= 2048), then every layer's routing (ids, weights, the router's
    # pair order and offsets), rounded up to 256 bytes
    assert need == (20480 + 2 * 2560 * 8 + 2 * 2048 * 8 + 3 * 48 * 8 * 4 + 1025 * 4 + 255) // 256 * 256
    assert all(mq.stack_workspace_size(H) == need for H in (256, 512, 1024))
    assert mq.stack_workspace_size(100) == 0
    k = 8

    def call(layers=None, L=3, k=k, flags=0, logits=A, h=A, h_all=None, hq=None, hd=None, ws=A, ws_bytes=need):
        layers = (mq._CExperts * max(L, 1))(*[_experts(E=128) for _ in range(max(L, 1))]) if layers is None else layers
        return f(layers, L, logits, k, flags, h, h_all, hq, hd, ws, ws_bytes, None)

    def stack(*exs):
        return (mq._CExperts * len(exs))(*exs)

    assert f(None, 3, A, k, 0, A, None, None, None, A, need, None) == mq.ERR_INVALID_ARG
    assert call(L=0) == mq.ERR_INVALID_ARG
    assert call(flags=4) == mq.ERR_INVALID_ARG                                  # unknown flag
    assert call(logits=None) == mq.ERR_INVALID_ARG
    assert call(h=A + 4) == mq.ERR_INVALID_ARG                                  # h not 16-byte aligned
    assert call(hq=A) == mq.ERR_INVALID_ARG                                     # hq_all without hd_all
    assert call(k=0) == mq.ERR_INVALID_ARG
    assert call(layers=stack(_experts(E=4), _experts(E=4)), L=2, k=5) == mq.ERR_INVALID_ARG  # k > E
    assert call(layers=stack(_experts(E=128), _experts(E=64)), L=2) == mq.ERR_INVALID_ARG  # mixed shapes
    assert call(layers=stack(_experts(E=128), _experts(E=128, ptr=A + 8)), L=2) == mq.ERR_INVALID_ARG
    assert call(L=49) == mq.ERR_UNSUPPORTED                                     # above the layer limit
    assert call(k=9) == mq.ERR_UNSUPPORTED                                      # one quad per expert: k <= 8
    assert call(layers=stack(_experts(E=128, I=256)), L=1) == mq.ERR_UNSUPPORTED
    assert call(layers=stack(_experts(E=128, H=4096)), L=1) == mq.ERR_UNSUPPORTED
    assert call(ws=None) == mq.ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == mq.ERR_WORKSPACE
    assert call(ws=A + 64) == mq.ERR_WORKSPACE                                  # ws not 256-byte aligned


def test_gemv_and_debug_validation(lib):
    assert lib.moe_q4_gemv(A, A, 512, 2048, A, A, 65, A, None) == mq.ERR_UNSUPPORTED
    assert lib.moe_q4_gemv(A, A, 512, 100, A, A, 1, A, None) == mq.ERR_UNSUPPORTED
    assert lib.moe_q4_gemv(None, A, 512, 2048, A, A, 1, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_debug_block_dots(A, 16, 2048, A, 1, 1, A, None) == mq.ERR_UNSUPPORTED  # down walk K
    ex = _experts()
    assert lib.moe_q4_debug_prefill_dots(ctypes.byref(ex), A, A, 4, 2, A, A, 2, A, A, 1 << 30,
                                         None) == mq.ERR_INVALID_ARG


def test_prefill_a16_validation(lib):
    f = lib.moe_q4_prefill_a16
    T, k = 4, 2
    need = mq.prefill_a16_workspace_size(T, k, 2048, 512)
    a = lambda v: (v + 255) // 256 * 256
    assert need == a(T * 2048 * 2) + a(T * k * 512 * 2) + a(T * k * 2048 * 4)
    ex = _experts()

    def call(ex=ex, T=T, k=k, flags=0, x=A, ws=A, ws_bytes=need):
        return f(ctypes.byref(ex), x, T, k, A, A, A, A, flags, A, ws, ws_bytes, None)

    assert call(x=None) == mq.ERR_INVALID_ARG
    assert call(x=A + 4) == mq.ERR_INVALID_ARG             # x not 16-byte aligned
    assert call(flags=mq.QUANT_RMSNORM) == mq.ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == mq.ERR_WORKSPACE
    assert call(ws=None) == mq.ERR_WORKSPACE
    assert call(ex=_experts(E=2000)) == mq.ERR_UNSUPPORTED
    assert f(ctypes.byref(ex), None, 0, k, None, None, None, None, 0, None, None, 0, None) == mq.OK  # T == 0


def test_router_logits_validation(lib):
    f = lib.moe_q4_router_logits
    assert f(None, 1, 2048, A, 128, 0, A, None) == mq.ERR_INVALID_ARG
    assert f(A, 1, 2048, None, 128, 0, A, None) == mq.ERR_INVALID_ARG
    assert f(A, 1, 2048, A, 128, 0, None, None) == mq.ERR_INVALID_ARG
    assert f(A + 4, 1, 2048, A, 128, 0, A, None) == mq.ERR_INVALID_ARG   # x not 16-byte aligned
    assert f(A, 1, 2040, A, 128, 0, A, None) == mq.ERR_INVALID_ARG       # H % 32
    assert f(A, 1, 2048, A, 0, 0, A, None) == mq.ERR_INVALID_ARG         # E < 1
    assert f(A, -1, 2048, A, 128, 0, A, None) == mq.ERR_INVALID_ARG      # T < 0
    assert f(A, 1, 2048, A, 128, 4, A, None) == mq.ERR_INVALID_ARG       # unknown flag
    assert f(A, 1, 32768, A, 128, 0, A, None) == mq.ERR_UNSUPPORTED      # H above the limit
    assert f(A, 1, 2048, A, 2000, 0, A, None) == mq.ERR_UNSUPPORTED      # E above the limit
    assert f(None, 0, 2048, None, 128, 0, None, None) == mq.OK           # T == 0: no-op


def test_probe_validation(lib):
    """The measurement probes reject bad arguments before any launch."""
    assert lib.moe_q4_probe_read(None, 1024, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_read(A, 0, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_read(A, 1000, A, None) == mq.ERR_INVALID_ARG      # not a multiple of 16
    assert lib.moe_q4_probe_read(A + 8, 1024, A, None) == mq.ERR_INVALID_ARG  # misaligned
    assert lib.moe_q4_probe_read(A, 1024, None, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_mfma_i8(0, 4, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_mfma_i8(8, 0, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_mfma_i8(8, 4, None, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_w4a8_step(0, 4, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_w4a8_step(8, 0, A, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_w4a8_step(8, 4, None, None) == mq.ERR_INVALID_ARG
    assert lib.moe_q4_probe_w4a8_step(8, 4, A + 2, None) == mq.ERR_INVALID_ARG


def test_no_fallback_without_library(tmp_path, monkeypatch):
    import importlib
    import sys
    monkeypatch.setattr(mq, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        mq.load_library(str(tmp_path / "missing.so"))
    importlib.reload(sys.modules["quantized_moe_q4_amd"])
