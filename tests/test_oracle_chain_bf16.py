"""Pins for the oracle's elementwise chain and its bf16 rounding (CPU only).

* ADD and MUL are exactly rounded fp32 ops, so they must equal numpy's
  float32 arithmetic bit for bit (the Triton tutorial page's closing check
  prints a max difference of 0.0 for its add; see tests/golden).
* The C3 chain 0.5 * GELU(x + 1) ("Lecture 6: GPU Kernels and Triton",
  section 1.1: three consecutive elementwise ops) is pinned against torch's
  double GELU applied to numpy's fp32 x + 1, rounded by numpy.
* fp32 -> bf16 nearest-even is pinned bit for bit against torch's own
  conversion over random bit patterns and hand-picked ties.
* ReLU (an op of the chain and an epilogue of the Linear kernel) is exact:
  x for x > 0, +0 otherwise, NaN kept, as torch's relu.
"""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle

GOLDEN = Path(__file__).parent / "golden"
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_bf16_bits(xf32):
    return torch.from_numpy(np.ascontiguousarray(xf32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_add_and_mul_are_exact_fp32_ops():
    gold = json.loads((GOLDEN / "add_exactness.json").read_text())
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32),
                        np.float32([0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38, np.inf])])
    for kind, s, ref in [(oracle.OP_ADD_SCALAR, 1.0, x + np.float32(1.0)),
                         (oracle.OP_ADD_SCALAR, -0.3, x + np.float32(-0.3)),
                         (oracle.OP_MUL_SCALAR, 0.5, x * np.float32(0.5)),
                         (oracle.OP_MUL_SCALAR, 3.7, x * np.float32(3.7))]:
        got = oracle.chain(x, [(kind, s)])
        fin = np.isfinite(ref)
        assert float(np.max(np.abs(got[fin] - ref[fin]))) == gold["max_abs_difference"]
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_c3_chain_against_torch():
    rng = np.random.default_rng(12)
    x = rng.uniform(-6, 6, 300_000).astype(np.float32)
    ops = [(oracle.OP_ADD_SCALAR, 1.0), (oracle.OP_GELU_TANH, 0.0), (oracle.OP_MUL_SCALAR, 0.5)]
    got = oracle.chain(x, ops)
    t1 = x + np.float32(1.0)
    g = torch.nn.functional.gelu(torch.from_numpy(t1.astype(np.float64)),
                                 approximate="tanh").numpy()
    # torch's literal form is accurate to ~1e-9 relative down to -4.5; beyond
    # that compare with the erf-free identity only through the other pins.
    keep = t1 > -4.5
    ref = g.astype(np.float32) * np.float32(0.5)
    rel = np.abs(got[keep] - ref[keep]) / np.maximum(np.abs(ref[keep]), 1e-30)
    assert rel.max() < 1.2e-7                     # within one fp32 rounding
    assert np.mean(got[keep] == ref[keep]) > 0.9999


def test_chain_equals_ops_applied_one_by_one():
    rng = np.random.default_rng(13)
    x = rng.uniform(-6, 6, 100_000).astype(np.float32)
    ops = [(oracle.OP_ADD_SCALAR, 1.0), (oracle.OP_GELU_TANH, 0.0), (oracle.OP_MUL_SCALAR, 0.5)]
    fused = oracle.chain(x, ops)
    step = x
    for op in ops:
        step = oracle.chain(step, [op])
    assert np.array_equal(fused.view(np.uint32), step.view(np.uint32))


def test_invalid_op_lists_are_rejected():
    x = np.zeros(4, np.float32)
    with pytest.raises(ValueError):
        oracle.chain(x, [])
    with pytest.raises(ValueError):
        oracle.chain(x, [(9, 1.0)])


def test_bf16_rounding_matches_torch_on_random_bits():
    rng = np.random.default_rng(14)
    bits = rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got = oracle.f32_to_bf16(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    gn = oracle.bf16_to_f32(got[nan])
    assert np.all(np.isnan(gn))


@pytest.mark.parametrize("f32_bits,bf16_bits", [
    (0x3F808000, 0x3F80),   # tie, kept half even -> down
    (0x3F818000, 0x3F82),   # tie, kept half odd -> up
    (0x3F808001, 0x3F81),   # just above the tie -> up
    (0x3F807FFF, 0x3F80),   # just below the tie -> down
    (0x7F7FFFFF, 0x7F80),   # max finite rounds to +inf
    (0xFF7FFFFF, 0xFF80),   # and to -inf
    (0x00008000, 0x0000),   # subnormal tie to even (zero)
    (0x00018000, 0x0002),   # subnormal tie to even (up)
    (0x80000000, 0x8000),   # -0 stays -0
    (0x7F800000, 0x7F80),   # inf
])
def test_bf16_rounding_hand_cases(f32_bits, bf16_bits):
    x = np.array([f32_bits], np.uint32).view(np.float32)
    assert int(oracle.f32_to_bf16(x)[0]) == bf16_bits
    assert int(_torch_bf16_bits(x)[0]) == bf16_bits


def test_bf16_nan_stays_nan():
    for b in (0x7F800001, 0x7FC00000, 0xFFFFFFFF, 0x7F810000):
        x = np.array([b], np.uint32).view(np.float32)
        y = oracle.f32_to_bf16(x)
        assert np.isnan(oracle.bf16_to_f32(y))[0]


def test_bf16_widening_is_exact():
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = oracle.bf16_to_f32(allbits)
    assert np.array_equal(w.view(np.uint32), allbits.astype(np.uint32) << 16)


def test_relu_is_exact_and_keeps_nan():
    rng = np.random.default_rng(14)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.float32([0.0, -0.0, 1e-40, -1e-40, np.inf, -np.inf, np.nan])])
    got = oracle.chain(x, [(oracle.OP_RELU, 0.0)])
    ref = torch.relu(torch.from_numpy(x)).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(x))
    ok = ~np.isnan(x)
    assert np.array_equal(got[ok], ref[ok])
    assert np.all(np.signbit(got[ok]) == False)   # -0 and negatives give +0  # noqa: E712
    # a chain with ReLU inside: 2 * relu(x - 1), each op an fp32 kernel
    two = oracle.chain(x[ok], [(oracle.OP_ADD_SCALAR, -1.0), (oracle.OP_RELU, 0.0),
                               (oracle.OP_MUL_SCALAR, 2.0)])
    want = np.maximum(x[ok] + np.float32(-1.0), np.float32(0.0)) * np.float32(2.0)
    assert np.array_equal(two, want)
