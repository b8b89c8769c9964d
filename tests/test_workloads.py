"""The seeded input generators: determinism and the configured distributions (CPU)."""
import numpy as np

from memory_bound_elementwise_fk_amd import workloads as w


def test_deterministic_and_thread_independent():
    a = w.draw(3 * w.CHUNK + 17, seed=0, threads=1)
    b = w.draw(3 * w.CHUNK + 17, seed=0, threads=5)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = w.draw(1000, seed=1)
    assert not np.array_equal(a[:1000], c)


def test_chunks_can_be_drawn_alone():
    full = w.draw(2 * w.CHUNK, seed=0)
    second = w.draw(w.CHUNK, seed=0, first_chunk=1)
    assert np.array_equal(full[w.CHUNK:], second)


def test_c1_c3_distributions():
    x1 = w.make_input("C1")
    assert x1.shape == (1_000_003,) and x1.dtype == np.float32
    assert abs(x1.mean()) < 5e-3 and abs(x1.std() - 1) < 5e-3
    x3 = w.make_input("C3")
    assert x3.shape == (8_388_608,)
    assert x3.min() >= -6 and x3.max() <= 6 and abs(x3.mean()) < 1e-2


def test_c2_shifted_rows():
    x = w.make_input("C2")
    assert x.shape == (4096, 1000)
    shifted = x[::16]
    others = np.delete(x, np.s_[::16], axis=0)
    assert abs(shifted.mean() - 80) < 0.05 and abs(others.mean()) < 0.05
    assert abs(others.std() - 3) < 0.01


def test_c4_mask_and_bf16_storage():
    x = w.make_input("C4", rows=512)
    assert x.dtype == np.uint16 and x.shape == (512, 4096)
    masked = x == w.BF16_MINUS_1E4
    assert 0.009 < masked.mean() < 0.011
    vals = (x[~masked].astype(np.uint32) << 16).view(np.float32)
    assert abs(vals.std() - 8) < 0.05
    # the first rows equal the first rows of a larger draw
    y = w.make_input("C4", rows=16)
    assert np.array_equal(x[:16], y)


def test_bf16_bits_round_trip_torch():
    f = np.float32([1.0, -2.5, 3.0e38, -1e4])
    bits = w.f32_to_bf16_bits(f)
    assert list(bits) == [0x3F80, 0xC020, 0x7F62, 0xC61C]
