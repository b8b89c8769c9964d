"""Tolerances of the parity tests, written once.

* fp32 tanh-GELU and the fp32 chain: |y - r| <= 1e-5 |r|, with an absolute
  floor of FLT_MIN (1.18e-38) that only matters where the result itself is
  subnormal or zero; NaN where the oracle has NaN, infinities equal.
* fp32 softmax: |y - r| <= 2e-6.
* bf16 outputs: within one bf16 ulp of the oracle's fp32 result rounded to
  bf16 (distance of the bit patterns in the monotone integer order).
* Integer / index / masking results: bit-exact.
"""
import numpy as np

GELU_REL = 1e-5
GELU_FLOOR = np.float32(np.finfo(np.float32).tiny)
SOFTMAX_ABS = 2e-6
BF16_ULPS = 1


def ordered_bf16(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers whose order is the numeric order."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ordered_f32(a: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def _nan_pattern_equal(got_nan, ref_nan, what):
    bad = np.flatnonzero(got_nan != ref_nan)
    assert bad.size == 0, f"{what}: NaN pattern differs at {bad[:8]}"


def assert_gelu_f32(got: np.ndarray, ref: np.ndarray, what: str = "gelu") -> None:
    got = np.asarray(got, np.float32).ravel()
    ref = np.asarray(ref, np.float32).ravel()
    gn, rn = np.isnan(got), np.isnan(ref)
    _nan_pattern_equal(gn, rn, what)
    ok = ~rn
    g, r = got[ok].astype(np.float64), ref[ok].astype(np.float64)
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), f"{what}: infinities differ"
    err = np.abs(g[~inf] - r[~inf])
    lim = GELU_REL * np.abs(r[~inf]) + float(GELU_FLOOR)
    bad = np.flatnonzero(err > lim)
    assert bad.size == 0, (f"{what}: {bad.size} elements beyond 1e-5 rel; worst rel "
                           f"{(err / np.maximum(np.abs(r[~inf]), 1e-38)).max():.3e}")


def assert_softmax_f32(got: np.ndarray, ref: np.ndarray, what: str = "softmax") -> None:
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    _nan_pattern_equal(np.isnan(got), np.isnan(ref), what)
    ok = ~np.isnan(ref)
    err = np.abs(got[ok].astype(np.float64) - ref[ok].astype(np.float64))
    assert err.size == 0 or err.max() <= SOFTMAX_ABS, f"{what}: max abs err {err.max():.3e}"


def assert_bf16(got: np.ndarray, ref: np.ndarray, what: str = "bf16") -> None:
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    gn = (got & 0x7FFF) > 0x7F80
    rn = (ref & 0x7FFF) > 0x7F80
    _nan_pattern_equal(gn, rn, what)
    ok = ~rn
    d = np.abs(ordered_bf16(got[ok]) - ordered_bf16(ref[ok]))
    assert d.size == 0 or d.max() <= BF16_ULPS, (
        f"{what}: {(d > BF16_ULPS).sum()} elements beyond one bf16 ulp (max {d.max()})")


def max_rel(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ok = np.isfinite(ref) & (ref != 0)
    return float((np.abs(got[ok] - ref[ok]) / np.abs(ref[ok])).max()) if ok.any() else 0.0
