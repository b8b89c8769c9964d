"""Exact-result pins for the oracle's row softmax (CPU only).

The definition is that of the "CS336 lecture 6" notes, section 5.2: per
row, y_j = exp(x_j - m) / sum_k exp(x_k - m) with m the row max. Here it is
evaluated in 60-digit decimal arithmetic from the stored fp32 / bf16 inputs
(exact for an fp32 comparison), on rows like the workloads': fp32 rows of
1000 values ~ N(0, 3^2), some shifted by +80; bf16 rows ~ 8 N(0, 1) with
entries set to -9984 (bf16(-1e4)). The oracle sums in double and rounds
once to fp32, so its results lie within one fp32 ulp of the exact values
(half an ulp from the final rounding, a little more from the double
arithmetic), and almost all are the exact value correctly rounded.
"""
from decimal import Decimal, localcontext

import numpy as np

import oracle
from memory_bound_elementwise_fk_amd import workloads as wl

def softmax_exact(row) -> list:
    with localcontext() as ctx:
        ctx.prec = 60
        xs = [Decimal(float(v)) for v in row]
        m = max(xs)
        es = [(v - m).exp() for v in xs]
        s = sum(es)
        return [e / s for e in es]


def _round_f32(d: Decimal) -> np.float32:
    """Nearest fp32 to a positive decimal (via the two fp32 neighbours of its double)."""
    f = np.float32(float(d))
    lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
    return min((lo, f, hi), key=lambda c: abs(Decimal(float(c)) - d))


def _check_f32(x, got):
    n_exact = 0
    for r in range(x.shape[0]):
        ex = softmax_exact(x[r])
        for j in range(x.shape[1]):
            g = got[r, j]
            if ex[j] < Decimal("1e-45"):
                assert g == 0 or abs(Decimal(float(g)) - ex[j]) <= Decimal("1.5e-45")
                continue
            ulp = Decimal(float(np.spacing(np.float32(float(ex[j])))))
            assert abs(Decimal(float(g)) - ex[j]) <= ulp, (r, j, float(g), float(ex[j]))
            n_exact += g == _round_f32(ex[j])
    return n_exact


def test_fp32_rows_with_shift_match_exact():
    x = wl.draw(4 * 1000, seed=3, scale=3.0, row_len=1000, row_period=2, row_shift=80.0
                ).reshape(4, 1000)
    assert x[0].mean() > 70 and abs(x[1].mean()) < 1  # rows 0 and 2 carry the +80
    got = oracle.softmax_rows(x)
    n_exact = _check_f32(x, got)
    assert n_exact >= 0.999 * x.size


def test_bf16_rows_with_masked_entries_match_exact():
    rng = np.random.default_rng(5)
    xf = (8.0 * rng.standard_normal((3, 512))).astype(np.float32)
    xf[rng.random((3, 512)) < 0.05] = -1e4
    xb = wl.f32_to_bf16_bits(xf)
    assert np.any(xb == 0xC61C)  # -9984, bf16(-1e4)
    got = oracle.softmax_rows(xb)
    xw = (xb.astype(np.uint32) << 16).view(np.float32)  # the stored bf16 values, widened
    n_equal = 0
    for r in range(3):
        ex = softmax_exact(xw[r])
        for j in range(512):
            want = np.float32(_round_f32(ex[j])) if ex[j] >= Decimal("1e-45") else np.float32(0)
            want_b = wl.f32_to_bf16_bits(np.array([want], np.float32))[0]
            gb = int(got[r, j])
            # bf16 of the fp32 result: equal to bf16 of the correctly rounded fp32
            # value, or one bf16 ulp away where the two fp32 values straddle a tie
            assert abs(gb - int(want_b)) <= 1, (r, j, hex(gb), hex(int(want_b)))
            if xb[r, j] == 0xC61C:
                assert gb == 0  # masked entries are exactly 0
            n_equal += gb == int(want_b)
    assert n_equal >= 0.999 * xb.size
