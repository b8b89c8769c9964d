"""GPU parity of the fp32 -> bf16 store (round to nearest, ties to even;
NaN kept quiet with its sign and leading payload bits) on crafted values.

Every bf16 output of the library leaves the kernels through one packing
routine; these tests drive chosen fp32 values into it through the chain
entry point: a bf16 input of ones multiplied by an fp32 scalar
(``MUL_SCALAR``, 1 * s == s exactly, signed zeros, subnormals, infinities
and NaN payloads included) and stored as bf16. Each value goes through the
three store routes of the elementwise kernels -- whole 16-byte vectors,
the masked vectors and < 16-byte tail of the ragged last tile, and the
one-element-per-lane kernel for unaligned pointers -- and every output
must equal, bit for bit, both the hand-written pattern below and the
oracle's conversion of the same fp32 value. The rule is not on the pages;
it is the nearest-even bf16 rounding the workloads' bf16 configurations
name (bit-exact for dtype conversion).
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from tests.gpu_util import DEV, guarded, guards_intact, to_host

pytestmark = pytest.mark.gpu

# (fp32 bits, bf16 bits): the expected result written out by hand
CASES = [
    # exact ties: the kept half even stays, odd rounds up to even
    (0x3F808000, 0x3F80), (0xBF808000, 0xBF80), (0x40408000, 0x4040),
    (0x3F818000, 0x3F82), (0xBF818000, 0xBF82), (0x4B7F8000, 0x4B80),
    (0x3FFF8000, 0x4000),   # tie on an odd mantissa carries into the exponent
    (0x00408000, 0x0040), (0x00418000, 0x0042),   # ties among subnormal results
    # near ties on either side
    (0x3F808001, 0x3F81), (0x3F807FFF, 0x3F80), (0x3F818001, 0x3F82),
    (0x3F817FFF, 0x3F81), (0xC2C9FFFF, 0xC2CA), (0xC2C97FFF, 0xC2C9),
    (0x3F800001, 0x3F80), (0x3F80FFFF, 0x3F81),
    # the largest finite values: up to infinity at and above the tie
    (0x7F7F7FFF, 0x7F7F), (0x7F7F8000, 0x7F80), (0x7F7FFFFF, 0x7F80),
    (0xFF7F7FFF, 0xFF7F), (0xFF7F8000, 0xFF80), (0xFF7FFFFF, 0xFF80),
    (0x7F7E8000, 0x7F7E), (0x7F7E8001, 0x7F7F),
    # fp32 subnormals
    (0x00000001, 0x0000), (0x80000001, 0x8000), (0x00008000, 0x0000),
    (0x00018000, 0x0002), (0x80018000, 0x8002), (0x00008001, 0x0001),
    (0x007FFFFF, 0x0080),   # the largest subnormal rounds up to the smallest normal
    (0x807F7FFF, 0x807F), (0x00400000, 0x0040), (0x007F8000, 0x0080),
    # signed zeros, infinities, the smallest normal
    (0x00000000, 0x0000), (0x80000000, 0x8000), (0x7F800000, 0x7F80),
    (0xFF800000, 0xFF80), (0x00800000, 0x0080), (0x80800000, 0x8080),
    # NaN: quiet, sign and leading payload bits kept
    (0x7FC00000, 0x7FC0), (0xFFC00000, 0xFFC0), (0x7FC12345, 0x7FC1),
    (0xFFE5A5A5, 0xFFE5), (0x7FFFFFFF, 0x7FFF), (0x7FC08000, 0x7FC0),
]

# 2 full tiles of 1024 bf16 values (128 lanes x 8), 3 masked vectors, a
# 5-element tail
N = 2 * 1024 + 3 * 8 + 5
ONE_BF16 = 0x3F80


def _f32(bits: int) -> float:
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def _run(x, scalar: float) -> np.ndarray:
    full, y = guarded(x.shape, torch.bfloat16)
    fk.fk_elementwise_chain(x, y, [(fk.FK_OP_MUL_SCALAR, scalar)])
    got = to_host(y)
    assert guards_intact(full, x.numel()), "chain wrote outside its output"
    return got


@pytest.fixture(scope="module")
def ones():
    base = torch.full((N + 1,), ONE_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return base[:N], base[1:]          # 16-byte aligned, and one element off


def test_oracle_agrees_with_the_hand_written_bits():
    f = np.array([c[0] for c in CASES], np.uint32).view(np.float32)
    want = np.array([c[1] for c in CASES], np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(f), want)


@pytest.mark.parametrize("f32_bits,bf16_bits", CASES,
                         ids=[f"{a:08X}->{b:04X}" for a, b in CASES])
def test_device_bf16_store_is_nearest_even(ones, f32_bits, bf16_bits):
    aligned, offset = ones
    s = _f32(f32_bits)
    want = int(oracle.f32_to_bf16(np.array([f32_bits], np.uint32).view(np.float32))[0])
    assert want == bf16_bits
    for x, route in ((aligned, "vector body + ragged tile"), (offset, "unaligned scalar kernel")):
        got = _run(x, s)
        bad = np.flatnonzero(got != bf16_bits)
        assert bad.size == 0, (f"{route}: fp32 0x{f32_bits:08X} stored as "
                               f"0x{int(got[bad[0]]):04X} at {bad[:4]}, want 0x{bf16_bits:04X}")


def test_device_bf16_store_random_patterns_bit_exact(ones):
    # values whose discarded half is drawn near the tie, over many exponents
    rng = np.random.default_rng(5)
    hi = rng.integers(0, 0x7F7F, 48, dtype=np.uint32)
    lo = (0x8000 + rng.integers(-2, 3, 48)).astype(np.uint32)
    sign = rng.integers(0, 2, 48, dtype=np.uint32) << 31
    bits = sign | (hi << 16) | lo
    aligned, _ = ones
    for b in bits:
        b = int(b)
        want = int(oracle.f32_to_bf16(np.array([b], np.uint32).view(np.float32))[0])
        got = _run(aligned, _f32(b))
        assert np.all(got == want), f"fp32 0x{b:08X}: got 0x{int(got[0]):04X}, want 0x{want:04X}"
