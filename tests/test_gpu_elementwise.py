"""GPU parity of the elementwise kernels against the CPU oracle (needs MI355X).

Every call goes through the C ABI (the ctypes binding). Inputs come from the
seeded generators; expected values only from the oracle.
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from memory_bound_elementwise_fk_amd import workloads as wl
from tests.gpu_util import CANARY_BITS, DEV, GUARD, guarded, guards_intact, random_input, tdtype, to_dev, \
    to_host
from tests.parity import assert_bf16, assert_gelu_f32

pytestmark = pytest.mark.gpu
T = oracle.default_threads()

C3 = list(wl.CHAIN_C3)


def run_gelu(x_np: np.ndarray, dt: str):
    xt = to_dev(x_np)
    full, y = guarded(x_np.shape, tdtype(dt))
    fk.fk_gelu_tanh(xt, y)
    got = to_host(y)
    assert guards_intact(full, x_np.size), "GELU wrote outside its output"
    return got


def check(dt, got, ref, what):
    if dt == "f32":
        assert_gelu_f32(got, ref, what)
    else:
        assert_bf16(got, ref, what)


# ------------------------------------------------------------------ GELU --
def test_c1_gelu_fp32_full_size():
    x = wl.make_input("C1")
    got = run_gelu(x, "f32")
    assert_gelu_f32(got, oracle.gelu_tanh(x, threads=T), "C1")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 15, 17, 255, 256, 257, 1023, 1025,
                               4095, 4096, 4097, 8191, 8192, 8193, 3 * 4096 + 5, 65536,
                               65536 + 7, 1_000_003])
def test_gelu_ragged_sizes(dt, n):
    x = random_input((n,), dt, 2.0, seed=n)
    got = run_gelu(x, dt)
    check(dt, got, oracle.gelu_tanh(x), f"gelu {dt} n={n}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("offx,offy", [(1, 1), (1, 2), (0, 3), (2, 0)])
def test_gelu_unaligned_pointers(dt, offx, offy):
    n = 5000
    x = random_input((n + 8,), dt, 2.0, seed=11)
    xt = to_dev(x)[offx:offx + n]
    full, ybuf = guarded((n + 8,), tdtype(dt))
    y = ybuf[offy:offy + n]
    fk.fk_gelu_tanh(xt, y)
    got = to_host(y)
    assert guards_intact(full, n + 8)
    check(dt, got, oracle.gelu_tanh(x[offx:offx + n]), f"gelu unaligned {offx},{offy}")
    pad = to_host(ybuf).view(np.uint16 if dt == "bf16" else np.uint32)
    # the elements of the buffer around the view are untouched canaries
    assert np.all(pad[:offy] == CANARY_BITS[dt]) and np.all(pad[offy + n:] == CANARY_BITS[dt])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gelu_in_place(dt):
    x = random_input((100_003,), dt, 3.0, seed=5)
    xt = to_dev(x)
    fk.fk_gelu_tanh(xt, xt)
    check(dt, to_host(xt), oracle.gelu_tanh(x), "gelu in place")


def test_gelu_fp32_special_values():
    x = np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, 6.0, 7.5, 1e20, 3.0e38, -30.0, -1e20,
                    -3.0e38, np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny, 1e-45,
                    -1e-45])
    got = run_gelu(x, "f32")
    ref = oracle.gelu_tanh(x)
    assert_gelu_f32(got, ref, "specials")
    bits = got.view(np.uint32)
    assert bits[0] == 0 and bits[1] == 0x80000000          # +0 -> +0, -0 -> -0
    assert got[2] == np.inf and bits[3] == 0x80000000       # -inf -> -0
    assert np.isnan(got[4])
    assert np.array_equal(got[5:9], x[5:9])                 # GELU(x) = x for x >= 6
    assert np.all(got[9:12] == 0) and np.all(np.signbit(got[9:12]))


def test_gelu_fp32_dense_sweep():
    # every 61st fp32 value in [-9.5, 12], plus a dense grid near zero
    lo, hi = np.float32(-9.5).view(np.uint32), np.float32(12.0).view(np.uint32)
    neg = np.arange(np.uint32(0x80000000), lo, 61, dtype=np.uint32).view(np.float32)
    pos = np.arange(0, hi, 61, dtype=np.uint32).view(np.float32)
    x = np.concatenate([neg, pos])
    got = run_gelu(x, "f32")
    assert_gelu_f32(got, oracle.gelu_tanh(x, threads=T), "dense sweep")


def test_gelu_fp32_far_negative_tail():
    # below -9.5 the result is tiny or subnormal; the floor FLT_MIN applies
    x = -np.geomspace(9.5, 40.0, 200_001).astype(np.float32)
    got = run_gelu(x, "f32")
    assert_gelu_f32(got, oracle.gelu_tanh(x), "far negative")
    assert np.all(np.signbit(got))


def test_gelu_bf16_every_bit_pattern():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = run_gelu(x, "bf16")
    assert_bf16(got, oracle.gelu_tanh(x), "all bf16")


def test_c5b_gelu_bf16_full_size():
    x = wl.make_input("C5b")
    xt = to_dev(x)
    y = torch.empty_like(xt)
    fk.fk_gelu_tanh(xt, y)
    got = to_host(y)
    del xt, y
    assert_bf16(got, oracle.gelu_tanh(x, threads=T), "C5b")


def _sample_indices(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(5000),
                                     np.arange(n - 5000, n)]))


def test_gelu_bf16_beyond_one_launch_grid():
    # 2^34 + 1001 bf16 elements (32 GiB per tensor): more tiles than one
    # launch's 2^31 work-items, so the kernel strides over tiles; checked on
    # sampled outputs (random, the first tiles, the ragged tail)
    n = (1 << 34) + 1001
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = torch.randn(n, dtype=torch.bfloat16, device=DEV, generator=gen).mul_(3)
    y = torch.empty_like(x)
    fk.fk_gelu_tanh(x, y)
    it = torch.from_numpy(_sample_indices(n, 6)).to(DEV)
    xs, ys = wl.from_torch(x[it]), wl.from_torch(y[it])
    del x, y
    torch.cuda.empty_cache()
    assert_bf16(ys, oracle.gelu_tanh(xs), "GELU bf16 2^34 + 1001, sampled")


def test_chain_fp32_beyond_one_launch_grid():
    # 2^33 + 3 fp32 elements (32 GiB per tensor): the fp32 tiles stride too
    n = (1 << 33) + 3
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    x = torch.rand(n, dtype=torch.float32, device=DEV, generator=gen).mul_(12).sub_(6)
    y = torch.empty_like(x)
    fk.fk_elementwise_chain(x, y, C3)
    it = torch.from_numpy(_sample_indices(n, 10)).to(DEV)
    xs, ys = wl.from_torch(x[it]), wl.from_torch(y[it])
    del x, y
    torch.cuda.empty_cache()
    assert_gelu_f32(ys, oracle.chain(xs, C3), "chain fp32 2^33 + 3, sampled")


# ----------------------------------------------------------------- chain --
def test_c3_chain_fused_full_size_and_unfused_equal():
    x = wl.make_input("C3")
    xt = to_dev(x)
    full, y = guarded(x.shape, torch.float32)
    fk.fk_elementwise_chain(xt, y, C3)
    got = to_host(y)
    assert guards_intact(full, x.size)
    assert_gelu_f32(got, oracle.chain(x, C3, threads=T), "C3 fused")
    # the same three ops as three kernels through fp32 intermediates
    t1, t2, t3 = torch.empty_like(xt), torch.empty_like(xt), torch.empty_like(xt)
    fk.fk_elementwise_chain(xt, t1, C3[:1])
    fk.fk_elementwise_chain(t1, t2, C3[1:2])
    fk.fk_elementwise_chain(t2, t3, C3[2:])
    unfused = to_host(t3)
    assert np.array_equal(unfused.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chain_add_mul_are_bit_exact(dt):
    x = random_input((70_001,), dt, 5.0, seed=3)
    ops = [(fk.FK_OP_ADD_SCALAR, -0.3), (fk.FK_OP_MUL_SCALAR, 3.7), (fk.FK_OP_ADD_SCALAR, 1.0)]
    got = to_host(fk.elementwise_chain(to_dev(x), ops))
    ref = oracle.chain(x, ops)
    assert np.array_equal(got.view(np.uint16 if dt == "bf16" else np.uint32),
                          ref.view(np.uint16 if dt == "bf16" else np.uint32))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chain_relu_is_bit_exact(dt):
    x = random_input((70_003,), dt, 3.0, seed=4)
    if dt == "f32":
        x[:6] = np.float32([0.0, -0.0, np.nan, np.inf, -np.inf, -1e-40])
    ops = [(fk.FK_OP_ADD_SCALAR, -0.5), (fk.FK_OP_RELU, 0.0), (fk.FK_OP_MUL_SCALAR, 2.0)]
    got = to_host(fk.elementwise_chain(to_dev(x), ops))
    ref = oracle.chain(x, ops)
    bits = np.uint16 if dt == "bf16" else np.uint32
    assert np.array_equal(got.view(bits), ref.view(bits))


# The last, ragged tile runs other code than the full tiles (whole vectors
# under a mask, then the < 16-byte tail one element per lane): the same
# inputs must give the same bits there as in the first, full tile.
# Workgroup tiles: fp32 64 lanes x 4 = 256 elements, bf16 128 lanes x 8 = 1024.
@pytest.mark.parametrize("dt,n", [("f32", 3 * 256 + 5 * 4 + 3), ("f32", 256 + 1),
                                  ("bf16", 3 * 1024 + 5 * 8 + 7), ("bf16", 1024 + 3)])
@pytest.mark.parametrize("op", ["gelu", "chain"])
def test_ragged_tile_matches_full_tile_bitwise(dt, n, op):
    tile = 256 if dt == "f32" else 1024
    rest = n % tile  # elements in the ragged tile
    specials = np.array([0.0, -0.0, 1.0, -1.0, 6.0, -3.0, -9.7, -30.0, 1e-30, np.inf, -np.inf,
                         np.nan], dtype=np.float32)
    xf = (np.random.default_rng(n).standard_normal(n) * 3.0).astype(np.float32)
    xf[:len(specials)] = specials
    xf[n - rest:] = xf[:rest]  # the ragged tile repeats the start of the first tile
    x = xf if dt == "f32" else wl.f32_to_bf16_bits(xf)
    xt = to_dev(x)
    full, y = guarded(x.shape, tdtype(dt))
    if op == "gelu":
        fk.fk_gelu_tanh(xt, y)
    else:
        fk.fk_elementwise_chain(xt, y, C3)
    got = to_host(y)
    assert guards_intact(full, n), f"{op} wrote outside its output"
    bits = got.view(np.uint32 if dt == "f32" else np.uint16)
    assert np.array_equal(bits[n - rest:], bits[:rest]), f"{op} {dt} n={n}: ragged tile differs"


# "scalar op, activation, scalar op" lists run a kernel with the kinds fixed
# at compile time when the data is 16-byte aligned; unaligned data runs the
# general op loop. Both must give the same bits, and match the oracle.
AAA = [(k0, k1, k2) for k0 in (fk.FK_OP_ADD_SCALAR, fk.FK_OP_MUL_SCALAR)
       for k1 in (fk.FK_OP_GELU_TANH, fk.FK_OP_RELU)
       for k2 in (fk.FK_OP_ADD_SCALAR, fk.FK_OP_MUL_SCALAR)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kinds", AAA, ids=["-".join(map(str, k)) for k in AAA])
def test_fixed_kind_chains_match_the_op_loop_and_the_oracle(dt, kinds):
    n = 3 * 4096 + 8 * 5 + 3   # full tiles, masked vectors, scalar tail
    # a positive trailing add: GELU(v) >= -0.17, so GELU(v) + 1.25 never cancels
    ops = [(kinds[0], 0.75), (kinds[1], 0.0), (kinds[2], 1.25)]
    flat = random_input((n + 1,), dt, 4.0, seed=sum(kinds) + (dt == "bf16"))
    if dt == "f32":
        flat[1:7] = np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, -30.0])
    base = to_dev(flat)
    aligned = base[:n].clone()               # 16-byte aligned: fixed-kind kernel
    x = flat[:n]
    full, y = guarded((n,), tdtype(dt))
    fk.fk_elementwise_chain(aligned, y, ops)
    got = to_host(y)
    assert guards_intact(full, n)
    check(dt, got, oracle.chain(x, ops), f"fixed-kind chain {kinds} {dt}")
    # the same values through the general op loop (unaligned input)
    yu = torch.empty(n + 1, dtype=tdtype(dt), device=DEV)[1:]
    xu = torch.empty(n + 1, dtype=tdtype(dt), device=DEV)[1:]
    xu.copy_(aligned)
    fk.fk_elementwise_chain(xu, yu, ops)
    gen = to_host(yu)
    bits = np.uint32 if dt == "f32" else np.uint16
    assert np.array_equal(got.view(bits), gen.view(bits)), "fixed-kind kernel differs from the op loop"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 4097, 50_001])
def test_chain_long_op_lists(dt, n):
    x = random_input((n,), dt, 2.0, seed=n + 1)
    ops = [(3, 0.0), (1, 0.25), (2, -1.5), (3, 0.0), (1, 2.0), (2, 0.5), (3, 0.0), (1, -0.125)]
    got = to_host(fk.elementwise_chain(to_dev(x), ops))
    check(dt, got, oracle.chain(x, ops), f"chain8 {dt} n={n}")


# ------------------------------------------------------------------ copy --
@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4095, 65536, 65536 * 4 + 13, 1 << 24])
@pytest.mark.parametrize("off", [0, 3])
def test_copy_is_bit_exact(nbytes, off):
    rng = np.random.default_rng(nbytes)
    src = rng.integers(0, 256, nbytes + 16, dtype=np.uint8)
    xs = torch.from_numpy(src).to(DEV)
    dst = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    x = xs[off:off + nbytes]
    y = dst[GUARD + off:GUARD + off + nbytes]
    fk.fk_copy(x, y)
    out = dst.cpu().numpy()
    assert np.array_equal(out[GUARD + off:GUARD + off + nbytes], src[off:off + nbytes])
    assert np.all(out[:GUARD + off] == 0xA5) and np.all(out[GUARD + off + nbytes:] == 0xA5)


def test_elementwise_runs_are_bitwise_reproducible():
    x = to_dev(random_input((300_001,), "f32", 3.0, seed=9))
    a = to_host(fk.gelu_tanh(x))
    b = to_host(fk.gelu_tanh(x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_stream_argument_is_honoured():
    x = to_dev(random_input((1 << 20,), "f32", 1.0, seed=4))
    s = torch.cuda.Stream()
    y = torch.empty_like(x)
    with torch.cuda.stream(s):
        fk.fk_gelu_tanh(x, y, stream=s)
    s.synchronize()
    assert_gelu_f32(y.cpu().numpy(), oracle.gelu_tanh(x.cpu().numpy()), "stream")
