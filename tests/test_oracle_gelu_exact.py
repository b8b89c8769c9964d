"""Exact-result pins for the oracle's tanh-GELU and its derivative (CPU only).

The definition is the tanh form of the "CS336 lecture 6" notes (kyc001),
section 4.2: GELU(x) = 0.5 x (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3).
Here it is evaluated literally -- the same expression, no rewriting -- in
150-digit decimal arithmetic (pi from Machin's formula, tanh from exp), so
the cancellation of 1 + tanh u for negative x costs nothing: the values are
exact for a double comparison. This pins the oracle where torch's float64
GELU cannot (it cancels below x ~ -4.5): down to x = -12, where GELU is
~1e-62 relative to x.

The oracle works in double from x: u carries a relative error of a few
2^-53 (the rounding of x^3, of the sum, of sqrt(2/pi) and of 0.044715 as
doubles), and exp(-2u) turns that into |2u| times as much, so the bound used
is |r - e| <= (8 |u(x)| + 8) 2^-53 |e| (|u| = 71 at x = -12: about 6e-14;
a wrong constant or a dropped term is off by 1e-3 or more).
"""
from decimal import Decimal, localcontext

import numpy as np

import oracle

PREC = 150  # digits; every evaluation runs in a local context of this precision


def _atan_inv(n: int) -> Decimal:
    """atan(1/n) by its Taylor series (n >= 2), in the current context."""
    x = Decimal(1) / n
    x2 = x * x
    term, total, k = x, x, 1
    eps = Decimal(10) ** (-PREC - 10)
    while True:
        term *= -x2
        k += 2
        d = term / k
        if abs(d) < eps:
            return total
        total += d


with localcontext() as _ctx:
    _ctx.prec = PREC + 10
    PI = 16 * _atan_inv(5) - 4 * _atan_inv(239)  # Machin
    C = (Decimal(2) / PI).sqrt()
A = Decimal("0.044715")


def _tanh(u: Decimal) -> Decimal:
    e = (2 * u).exp()
    return (e - 1) / (e + 1)


def gelu_exact(x: float) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = PREC
        X = Decimal(x)  # the double's exact value
        u = C * (X + A * X ** 3)
        return Decimal("0.5") * X * (1 + _tanh(u))


def gelu_grad_exact(x: float) -> Decimal:
    """d/dx of the literal expression: 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) u'."""
    with localcontext() as ctx:
        ctx.prec = PREC
        X = Decimal(x)
        u = C * (X + A * X ** 3)
        du = C * (1 + 3 * A * X ** 2)
        t = _tanh(u)
        return Decimal("0.5") * (1 + t) + Decimal("0.5") * X * (1 - t * t) * du


def _u(x):
    return 0.7978845608028654 * (x + 0.044715 * x ** 3)


def _bound(x):
    return (8 * np.abs(_u(x)) + 8) * 2.0 ** -53


XS = np.concatenate([np.linspace(-12.0, 12.0, 1201), [-0.75, -1e-3, 1e-3, 1e-20, -1e-20]])


def test_machin_pi():
    assert str(PI).startswith("3.14159265358979323846264338327950288419716939937510")


def test_gelu_matches_exact_literal_definition():
    r = oracle.gelu_tanh_f64(XS)
    for x, got in zip(XS, r):
        e = gelu_exact(float(x))
        if e == 0:
            assert got == 0
            continue
        rel = abs((Decimal(float(got)) - e) / e)
        assert rel <= Decimal(float(_bound(x))), (x, float(got), float(e), float(rel))


def test_gelu_far_negative_values():
    # the region torch cannot check: GELU(-9) ~ -1.3e-28, GELU(-12) ~ -1e-61
    for x in (-6.0, -7.5, -9.0, -10.5, -12.0):
        e = gelu_exact(x)
        got = oracle.gelu_tanh_f64(np.array([x]))[0]
        assert got < 0
        assert abs((Decimal(float(got)) - e) / e) <= Decimal(float(_bound(x)))


def test_gelu_fp32_is_the_exact_value_rounded():
    # fp32 results: the exact value rounded to nearest fp32 (ties cannot occur
    # here), i.e. within half an fp32 ulp of it
    x32 = np.linspace(-9.5, 9.5, 951).astype(np.float32)
    got = oracle.gelu_tanh(x32)
    for x, g in zip(x32, got):
        e = gelu_exact(float(x))
        if e == 0:
            continue
        half_ulp = Decimal(float(np.spacing(np.abs(np.float32(float(e)))))) / 2
        assert abs(Decimal(float(g)) - e) <= half_ulp * Decimal("1.0000001"), (x, g, float(e))


def test_gelu_grad_matches_exact_derivative():
    r = oracle.gelu_tanh_grad_f64(XS)
    for x, got in zip(XS, r):
        e = gelu_grad_exact(float(x))
        # near GELU's minimum (x ~ -0.75) the derivative crosses zero, so the
        # error there is absolute, of the size of its two terms' rounding
        tol = Decimal(float(_bound(x))) * (abs(e) + 1)
        assert abs(Decimal(float(got)) - e) <= tol, (x, float(got), float(e))
