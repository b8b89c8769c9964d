"""Exact-result pins for the oracle's LayerNorm (+ tanh-GELU) (CPU only).

LayerNorm over the last axis (the standard definition; "Lecture 6: GPU
Kernels and Triton", section 6.1 names the kernel without a formula):
mean, biased variance, y = (x - mean) / sqrt(var + eps) * gamma + beta,
optionally followed by the tanh-GELU of the "CS336 lecture 6" notes,
section 4.2. Evaluated here in 60-digit decimal arithmetic from the stored
fp32 inputs, on rows shifted far from zero (where a one-pass variance
cancels in floating point) and with random gamma and beta. The oracle works
in double and rounds once to fp32: within one fp32 ulp of the exact value,
almost always correctly rounded.
"""
from decimal import Decimal, localcontext

import numpy as np

import oracle
from tests.test_oracle_gelu_exact import gelu_exact


def layernorm_exact(row, g, b, eps: float, gelu: bool) -> list:
    with localcontext() as ctx:
        ctx.prec = 60
        xs = [Decimal(float(v)) for v in row]
        n = len(xs)
        mu = sum(xs) / n
        var = sum((v - mu) ** 2 for v in xs) / n
        rstd = 1 / (var + Decimal(eps)).sqrt()
        ts = [(v - mu) * rstd * Decimal(float(g[j])) + Decimal(float(b[j])) for j, v in enumerate(xs)]
    # the GELU of the exact affine value: its own 150-digit evaluation of the
    # value rounded to double (the oracle's GELU input is a double as well)
    return [gelu_exact(float(t)) if gelu else t for t in ts]


def test_layernorm_matches_exact():
    rng = np.random.default_rng(17)
    rows, cols = 4, 300
    x = (3.0 * rng.standard_normal((rows, cols))).astype(np.float32)
    x += np.float32(80.0) * (np.arange(rows, dtype=np.float32)[:, None] % 2)
    g = (1.0 + 0.25 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.5 * rng.standard_normal(cols)).astype(np.float32)
    for gelu in (False, True):
        got = oracle.layernorm_rows(x, g, b, eps=1e-5, gelu=gelu)
        n_close = 0
        for r in range(rows):
            ex = layernorm_exact(x[r], g, b, 1e-5, gelu)
            for j in range(cols):
                e = ex[j]
                if e == 0:
                    assert got[r, j] == 0
                    continue
                ulp = Decimal(float(np.spacing(np.abs(np.float32(float(e))))))
                d = abs(Decimal(float(got[r, j])) - e)
                assert d <= ulp, (gelu, r, j, float(got[r, j]), float(e))
                n_close += d <= ulp / 2 * Decimal("1.000001")
        assert n_close >= 0.995 * x.size
