"""Tolerance checks of a device result against the oracle -- test infrastructure.

Projection (per output, fp32 before bf16 rounding):
    |y_dev - y_oracle| <= tol * sum_k |D[n,k] * x[r,k]|,   tol = 1e-3,
with y_oracle the fp64 sum.  bf16 outputs: the device's bf16 must be the
round-to-nearest-even of its own fp32 result (bit exact), and within one bf16
ulp (distance of the ordered bit patterns) of the oracle's bf16 for every
output whose oracle value is not near cancellation:
    |y_oracle| >= 2^-12 * sum_k |D[n,k] * x[r,k]|.
Below that band two correct fp32 summation orders may straddle several bf16
steps, so only the fp32 bound applies there; those outputs are counted
("bf16_exempt") and printed with every check.

Gate/up pair o = silu(g) * u: first-order propagation of the per-projection
bound (|silu'| <= 1.1), plus 2^-20 |o| for the fp32 evaluation of silu:
    |o_dev - o| <= 1.1 tg (|u| + tu) + |silu(g)| tu + 2^-20 |o|,
    tg = tol * sum|D_g x|,  tu = tol * sum|D_u x|;
bf16 within one ulp wherever |o| >= 2^-12 (1.1 sum|D_g x| |u| + |silu(g)| sum|D_u x|).
"""
from __future__ import annotations

import numpy as np
import torch

TOL = 1e-3


def bf16_bits_of(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126), -126)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


BAND = 2.0 ** -12


def _bf16_checks(out32, out16, ref, ref16, band, label):
    """band: fp64 per output; bf16 <= 1 ulp is enforced where |ref| >= band."""
    stats = {}
    if out16 is None:
        return stats
    own = bf16_bits_of(out32)
    nbad_own = int(np.sum(own != out16))
    assert nbad_own == 0, "%s: %d bf16 outputs differ from RNE of the same fp32 result" % (label, nbad_own)
    enforce = np.abs(ref) >= band
    dist = np.abs(_ordered(out16) - _ordered(ref16))
    nbad = int(np.sum(dist[enforce] > 1))
    assert nbad == 0, "%s: %d bf16 outputs more than 1 ulp from the oracle (max %d ulp) outside the cancellation band" % (
        label, nbad, int(dist[enforce].max()))
    stats["bf16_max_ulp"] = int(dist[enforce].max()) if enforce.any() else 0
    stats["bf16_exempt"] = int(np.sum(~enforce))
    stats["bf16_exempt_max_ulp"] = int(dist[~enforce].max()) if (~enforce).any() else 0
    return stats


def _report(label, stats):
    print("%s: %s" % (label, ", ".join("%s=%s" % (k, ("%.3g" % v) if isinstance(v, float) else v)
                                       for k, v in stats.items())))


def check_gemv(out32, out16, ref, absdot, ref16, tol=TOL, label="gemv"):
    """out32: device fp32 [rows, n]; out16: device bf16 bits or None; ref/absdot fp64; ref16 uint16."""
    out32 = np.asarray(out32, np.float32)
    err = np.abs(out32.astype(np.float64) - ref)
    bar = tol * absdot
    nbad = int(np.sum(~(err <= bar)))
    rel = err / np.where(absdot > 0, absdot, 1.0)
    assert nbad == 0, "%s: %d outputs exceed %g*sum|w*x| (max ratio %g)" % (label, nbad, tol, rel.max())
    stats = {"max_err_over_absdot": float(rel.max()), "n": int(out32.size)}
    stats.update(_bf16_checks(out32, out16, ref, ref16, BAND * absdot, label))
    _report(label, stats)
    return stats


def dual_bound(d: dict, tol=TOL) -> np.ndarray:
    g, u, o = d["g"], d["u"], d["o"]
    tg, tu = tol * d["abs_g"], tol * d["abs_u"]
    silu = g / (1.0 + np.exp(-g))
    return 1.1 * tg * (np.abs(u) + tu) + np.abs(silu) * tu + 2.0 ** -20 * np.abs(o)


def check_dual(out32, out16, d: dict, tol=TOL, label="dual"):
    out32 = np.asarray(out32, np.float32)
    err = np.abs(out32.astype(np.float64) - d["o"])
    bound = dual_bound(d, tol)
    nbad = int(np.sum(~(err <= bound)))
    assert nbad == 0, "%s: %d outputs exceed the propagated bound" % (label, nbad)
    stats = {"max_err_over_bound": float(np.max(err / np.where(bound > 0, bound, 1.0))), "n": int(out32.size)}
    g = d["g"]
    silu = g / (1.0 + np.exp(-g))
    band = BAND * (1.1 * d["abs_g"] * np.abs(d["u"]) + np.abs(silu) * d["abs_u"])
    stats.update(_bf16_checks(out32, out16, d["o"], d["o_bf16"], band, label))
    _report(label, stats)
    return stats
