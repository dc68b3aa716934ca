"""Helpers shared by the GPU tests: device upload of synthetic inputs and the
comparison rules (bit-exact integers, boundary-only Q8_0 code differences,
fp32 within 1e-3 x the oracle RMS)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import quantized_moe_q4_amd as mq

TOL_RMS = 1e-3  # max |gpu - oracle| <= 1e-3 * RMS(oracle)


def banner(msg: str):
    """Name the case before each GPU step, so a failing run says which one."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def experts_to_dev(es) -> mq.Experts:
    return mq.Experts(to_dev(es.gate_qs), to_dev(es.up_qs), to_dev(es.down_qs), to_dev(es.gate_d), to_dev(es.up_d),
                      to_dev(es.down_d))


def np_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close_rms(got: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL_RMS):
    ref64 = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref64 ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got.astype(np.float64) - ref64))) if ref.size else 0.0
    assert err <= tol * rms or (rms == 0.0 and err == 0.0), \
        f"{what}: max abs err {err:.3e} > {tol:g} x RMS {rms:.3e}"
    return err, rms


def to_pair_order(rows_sorted: np.ndarray, sorted_pairs: np.ndarray) -> np.ndarray:
    """Rows indexed by sorted position -> rows indexed by pair id."""
    out = np.zeros_like(rows_sorted)
    out[sorted_pairs] = rows_sorted
    return out


def check_requant(hq_gpu: np.ndarray, hd_gpu: np.ndarray, h_ref: np.ndarray, hq_ref: np.ndarray, hd_ref: np.ndarray,
                  what: str, max_frac: float = 1e-3):
    """Q8_0 codes of h: equal, except where the oracle's h/d sits at a rounding boundary.

    GPU and oracle compute h in fp32 from different summation orders, so a code
    may legitimately land on the other side of a half-integer; such a case is
    accepted only if |h/d - (m + 1/2)| < 1e-2 for an integer m and the codes
    differ by one.  Scales must agree to 1e-5 relative.
    """
    np.testing.assert_allclose(hd_gpu, hd_ref, rtol=1e-5, atol=0, err_msg=f"{what}: h scales")
    mism = hq_gpu != hq_ref
    n_mis = int(mism.sum())
    if n_mis:
        P, I = h_ref.shape
        d = np.repeat(hd_ref.astype(np.float64), 32, axis=1)
        rel = np.where(d > 0, h_ref.astype(np.float64) / np.where(d > 0, d, 1.0), 0.0)
        dist = np.abs(rel - (np.floor(rel) + 0.5))
        ok = (dist < 1e-2) & (np.abs(hq_gpu.astype(np.int32) - hq_ref.astype(np.int32)) == 1)
        bad = mism & ~ok
        assert not bad.any(), f"{what}: {int(bad.sum())} Q8_0 codes differ away from a rounding boundary"
        assert n_mis <= max(2, max_frac * hq_ref.size), f"{what}: {n_mis} boundary flips of {hq_ref.size}"
    return n_mis
