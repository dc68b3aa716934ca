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


U32 = 2.0 ** -24  # unit roundoff of fp32 (round to nearest)
SILU_LIP = 1.1     # max |silu'(z)| = 1.0998...


def depth_decode(H: int) -> int:
    """Longest chain of fp32 roundings in a gate/up output of the decode row walk (rows.h): the product
    d_w/16 * d_a, H/256 fused multiply-adds per lane, then a 3-level tree over the row's 8 lanes."""
    return H // 256 + 4


def depth_prefill(H: int) -> int:
    """The prefill MFMA kernels: t = fl(isum d_w) (one rounding), then H/32 sequential fma into one
    accumulator per output."""
    return H // 32 + 1


def h_error_bound(g, u, sg, su, depth: int):
    """A rigorous bound on |h_gpu - h_exact| for h = silu(g) u, elementwise (fp64 arrays of the oracle's g, u,
    rounded to fp32, and of the block-magnitude sums sg, su).

    - g, u on the GPU: fp32 sums of the same block terms; with D roundings on the longest chain,
      |g_gpu - g| <= gamma_D * sum_b |d_w d_a isum_b| (Higham's recursive/tree summation bound,
      gamma_D = D u / (1 - D u)); the oracle's fp32 g adds u |g|.
    - silu is 1.1-Lipschitz, and on z <= -1 |silu'(z)| <= (1 + |z|) e^z, increasing in z, so over
      [g - dg, g + dg] entirely below -1 the slope is at most (1 - z_max) e^z_max, z_max = g + dg;
      the GPU's fp32 SwiGLU (an exponential accurate to a few ulp, or the base-2
      exponential of an argument rounded once, a reciprocal or a divide, two products) has a relative
      error at most (2 |g| + 8) u.
    - the oracle's h is rounded to fp32 once more (u |h|).
    """
    gs = g.astype(np.float64)
    ua = np.abs(u.astype(np.float64))
    gam = depth * U32 / (1.0 - depth * U32)
    dg = gam * sg + U32 * np.abs(gs)
    du = gam * su + U32 * ua
    zmax = gs + dg
    lip = np.where(zmax <= -1.0, np.minimum(SILU_LIP, (1.0 - zmax) * np.exp(np.clip(zmax, -700.0, -1.0))), SILU_LIP)
    # |silu| at the ends of [g - dg, g + dg] bounds it on the interval (silu is monotone on each side of its
    # minimum, where |silu| <= 0.28)
    sil_hi = np.maximum(np.abs(_silu(gs - dg)), np.abs(_silu(gs + dg)))
    sil_hi = np.maximum(sil_hi, np.where((gs - dg < -1.278) & (gs + dg > -1.278), 0.2785, 0.0))
    g = np.abs(gs)
    h = sil_hi * (ua + du)
    return lip * dg * (ua + du) + sil_hi * du + ((2.0 * g + 8.0) * U32 + 2 * U32) * (h + 1e-30)


def _silu(z):
    return z / (1.0 + np.exp(-np.clip(z, -700.0, 700.0)))


def check_requant(hq_gpu: np.ndarray, hd_gpu: np.ndarray, inter: dict, pairs: np.ndarray, depth: int, what: str,
                  quot_roundings: int = 2):
    """Q8_0 codes and scales of h (rows in pair order, for the given pair ids) against the oracle.

    The GPU computes h in fp32 along its own summation order, so the codes may differ from the oracle's only
    where the bound of h_error_bound makes both roundings possible.  With the GPU's own block scale d_g, the
    quotient h/d_g that its code rounds lies within W = (B + u|h|)/d_g + q u |h/d_g| of the oracle's
    r = h_o/d_g (q = roundings of the quotient: 1 for a division, 2 for a reciprocal and a product); the code
    must be rint of a value in [r - W, r + W] (clamped to +-127).  A scale may differ from the oracle's only by
    what the bound on the block's amax allows.  Returns a dict of counts for the report.
    """
    hq_o = inter["hq"][pairs]
    hd_o = inter["hd"][pairs].astype(np.float64)
    h_o = inter["h"][pairs].astype(np.float64)
    B = h_error_bound(inter["g"][pairs], inter["u"][pairs], inter["sg"][pairs], inter["su"][pairs], depth)
    P, I = h_o.shape
    nb = I // 32
    dg = hd_gpu.astype(np.float64)
    # scales: amax can move by at most the largest element bound of its block
    Bblk = (B + U32 * np.abs(h_o)).reshape(P, nb, 32).max(axis=2)
    amax_o = np.abs(h_o).reshape(P, nb, 32).max(axis=2)
    d_tol = (Bblk + U32 * amax_o) / 127.0 + U32 * (np.abs(dg) + hd_o)
    bad_d = np.abs(dg - hd_o) > d_tol
    assert not bad_d.any(), f"{what}: {int(bad_d.sum())} h block scales differ from the oracle beyond the bound"
    d_el = np.repeat(dg, 32, axis=1)
    safe = np.where(d_el > 0, d_el, 1.0)
    r = np.where(d_el > 0, h_o / safe, 0.0)
    W = np.where(d_el > 0, (B + U32 * np.abs(h_o)) / safe + quot_roundings * U32 * np.abs(r), 0.0)
    lo = np.clip(np.rint(r - W), -127, 127)
    hi = np.clip(np.rint(r + W), -127, 127)
    q = hq_gpu.astype(np.float64)
    bad = (q < lo) | (q > hi)
    assert not bad.any(), (f"{what}: {int(bad.sum())} Q8_0 codes of h outside the derived window "
                           f"(first at {np.argwhere(bad)[0].tolist()})")
    flips = int((hq_gpu != hq_o).sum())
    win = W[d_el > 0]
    return {"what": what, "elements": int(q.size), "flips": flips, "scales_differing": int((dg != hd_o).sum()),
            "window_max": float(win.max()) if win.size else 0.0,
            "window_median": float(np.median(win)) if win.size else 0.0}


def report(rec: dict):
    """Print a parity record and, when MOE_Q4_PARITY_REPORT names a file, append it there as a JSON line."""
    import json
    import os
    line = json.dumps(rec, sort_keys=True)
    print(f"[parity] {line}", flush=True)
    path = os.environ.get("MOE_Q4_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def oracle_threads() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def oracle_layer_all(es, xq, xd, ids, w, tokens=None, flags: int = 0, y0=None, hq_in=None, hd_in=None,
                     want_intermediates: bool = False):
    """oracle.moe_layer over the given tokens (default: all), split across host threads (the C call releases
    the GIL; threads write disjoint rows of shared outputs)."""
    import concurrent.futures

    import oracle
    T, k = ids.shape
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    y = np.zeros((T, es.H), np.float32) if y0 is None else np.ascontiguousarray(y0, np.float32).copy()
    inter = oracle.new_intermediates(T * k, es.I) if want_intermediates else None
    n = oracle_threads()
    chunks = [c for c in np.array_split(toks, n) if c.size]
    with concurrent.futures.ThreadPoolExecutor(len(chunks)) as pool:
        futs = [pool.submit(oracle.moe_layer, es, xq, xd, ids, w, tokens=c, flags=flags, y=y, hq_in=hq_in,
                            hd_in=hd_in, inter=inter) for c in chunks]
        for f in futs:
            f.result()
    return (y, inter) if want_intermediates else y
