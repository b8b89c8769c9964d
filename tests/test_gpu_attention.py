"""GPU parity of the FlashAttention forward kernel against the CPU oracle.
Needs an MI355X.

Tolerance (derived from the kernel's arithmetic; none is stated for
attention): |o - r| <= ulp_bf16(|r|) + 2^-8 max|v| per
(batch, head). O = sum_j p_j v_j / l. The kernel rounds p_j to bf16 before
the P V product (as the page's kernel rounds P to V's dtype): relative error
<= 2^-9 per weight, so at most 2^-9 max|v| after the division by l (the sum
l uses the unrounded p); the fp32 scores (128 bf16 products) move the
weights by ~1e-4 relative, far below that; the output rounding to bf16 adds
half an ulp on each side. 2^-8 leaves a factor 2 over the P rounding.
fp16 data (the pages benchmark fp16): the same argument with P rounded to
fp16 (2^-11 relative): |o - r| <= ulp_fp16(|r|) + 2^-10 max|v|.
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_fk_amd as fk
import oracle
from memory_bound_elementwise_fk_amd import workloads as wl
from tests.gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def bf16_ulp(r):
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126)))
    return np.exp2(e - 7)


def fp16_ulp(r):
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -14)))
    return np.exp2(e - 10)


def f64(a):
    """bf16 bits (uint16) or float16/float32 values -> float64."""
    return oracle.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def qkv(B, H, T, seed, d=128, dt="bf16"):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        a = rng.standard_normal((B, H, T, d)).astype(np.float32)
        out.append(a.astype(np.float16) if dt == "fp16"
                   else wl.f32_to_bf16_bits(a).reshape(B, H, T, d))
    return out


def check_rows(got_rows, ref_rows, v, what):
    """got_rows / ref_rows: {(b, h): [n, d]} of v's storage type."""
    fp16 = v.dtype == np.float16
    for key, ref in ref_rows.items():
        g = f64(got_rows[key])
        r = f64(ref)
        vmax = float(np.abs(f64(v[key[0], key[1]])).max())
        lim = (fp16_ulp(r) + 2.0 ** -10 * vmax) if fp16 else (bf16_ulp(r) + 2.0 ** -8 * vmax)
        err = np.abs(g - r)
        bad = np.flatnonzero(err > lim)
        assert bad.size == 0, f"{what} {key}: {bad.size} beyond tolerance, worst excess {(err - lim).max():.3e}"


def run(q, k, v, causal):
    o = fk.attention_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal)
    return to_host(o)


@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 2, 33), (2, 3, 128), (1, 2, 200), (1, 1, 513),
                                   (2, 2, 1000)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_attention_shapes(B, H, T, causal, dt):
    q, k, v = qkv(B, H, T, seed=B * 100 + H * 10 + T, dt=dt)
    got = run(q, k, v, causal)
    ref = oracle.attention(q, k, v, causal=causal)
    rows = {(b, h): np.arange(T) for b in range(B) for h in range(H)}
    check_rows({key: got[key[0], key[1]] for key in rows},
               {key: ref[key[0], key[1]] for key in rows}, v, f"B{B} H{H} T{T} causal={causal}")


# B H a multiple of 8: the workgroups go to the XCDs in groups of heads
# (1 head for full attention; for causal the largest divisor of B H / 8 up to
# 4: 1, 2, 3 and 4 below), a different order of the same (head, query block)
# pairs; every output row is checked, in several query blocks per head.
@pytest.mark.parametrize("B,H", [(1, 8), (2, 8), (3, 8), (1, 40), (4, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_head_groups(B, H, causal):
    T = 300
    q, k, v = qkv(B, H, T, seed=B * 1000 + H)
    got = run(q, k, v, causal)
    ref = oracle.attention(q, k, v, causal=causal)
    rows = {(b, h): np.arange(T) for b in range(B) for h in range(H)}
    check_rows({key: got[key[0], key[1]] for key in rows},
               {key: ref[key[0], key[1]] for key in rows}, v, f"B{B} H{H} T{T} causal={causal}")


def test_attention_strided_bthd_layout():
    # tensors stored as [B, T, H, d] and viewed as [B, H, T, d]
    B, H, T, d = 2, 4, 300, 128
    rng = np.random.default_rng(7)
    base = [wl.f32_to_bf16_bits(rng.standard_normal((B, T, H, d)).astype(np.float32))
            .reshape(B, T, H, d) for _ in range(3)]
    qt, kt, vt = (to_dev(a).permute(0, 2, 1, 3) for a in base)
    ot = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=DEV).permute(0, 2, 1, 3)
    fk.fk_attention_fwd(qt, kt, vt, ot, causal=True)
    got = to_host(ot.contiguous())
    q, k, v = (np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in base)
    ref = oracle.attention(q, k, v, causal=True)
    rows = {(b, h): np.arange(T) for b in range(B) for h in range(H)}
    check_rows({key: got[key[0], key[1]] for key in rows},
               {key: ref[key[0], key[1]] for key in rows}, v, "B,T,H,d layout")


@pytest.mark.parametrize("T", [128, 1024, 4096])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_attention_benchmark_grid_sampled(T, dt):
    # the pages' benchmark grid: B = 4, H = 32, d = 128
    B, H = 4, 32
    q, k, v = qkv(B, H, T, seed=T, dt=dt)
    for causal in (True, False):
        o = fk.attention_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal)
        rng = np.random.default_rng(T + causal)
        picks = {(int(b), int(h)): np.sort(rng.choice(T, min(T, 24), replace=False))
                 for b, h in zip(rng.integers(0, B, 4), rng.integers(0, H, 4))}
        ref = oracle.attention(q, k, v, causal=causal, rows=picks)
        got = {key: to_host(o[key[0], key[1]][torch.from_numpy(idx).to(DEV)])
               for key, idx in picks.items()}
        check_rows(got, ref, v, f"{dt} T={T} causal={causal}")


# B H T large enough that the launcher takes workgroups of 8 waves (256
# queries, one per CU: 2048 of them here, at least the four per CU that it
# needs for 8 waves on a 256-CU MI355X); T = 300 leaves the second query block ragged (44 queries) and the
# last key block partial. Every row of six heads is checked.
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_attention_eight_wave_workgroups(causal, dt):
    B, H, T = 8, 128, 300
    q, k, v = qkv(B, H, T, seed=31 + causal, dt=dt)
    o = fk.attention_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal)
    rng = np.random.default_rng(7 + causal)
    picks = {(int(b), int(h)): np.arange(T)
             for b, h in zip(rng.integers(0, B, 6), rng.integers(0, H, 6))}
    ref = oracle.attention(q, k, v, causal=causal, rows=picks)
    got = {key: to_host(o[key[0], key[1]]) for key in picks}
    check_rows(got, ref, v, f"8-wave {dt} causal={causal}")


# 8-wave workgroups over 1, 2, 3 and 4 key blocks (T = 40, 100, 150, 200:
# one query block each, 1024 workgroups, four per CU): the prologue's
# counted waits and the first iterations' loads differ with the number of
# key blocks. Every row of three heads, the last one included.
@pytest.mark.parametrize("T", [40, 100, 150, 200])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_eight_wave_few_key_blocks(T, causal):
    B, H = 8, 128
    q, k, v = qkv(B, H, T, seed=41 + T + causal)
    o = fk.attention_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal)
    picks = {(0, 0): np.arange(T), (3, 77): np.arange(T), (7, 127): np.arange(T)}
    ref = oracle.attention(q, k, v, causal=causal, rows=picks)
    got = {key: to_host(o[key[0], key[1]]) for key in picks}
    check_rows(got, ref, v, f"8-wave T={T} causal={causal}")


# 8-wave workgroups with B H not a multiple of 8 (one group of all heads,
# level by level): 1030 heads x 2 query blocks of 256 = 2060 workgroups, at
# least four per CU of a 256-CU MI355X, so both masks take 8 waves; every
# row of five heads, the last one included, is checked.
@pytest.mark.parametrize("causal", [True, False])
def test_attention_eight_wave_workgroups_ungrouped_heads(causal):
    B, H, T = 2, 515, 300
    q, k, v = qkv(B, H, T, seed=37 + causal)
    o = fk.attention_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal)
    picks = {(0, 0): np.arange(T), (0, 514): np.arange(T), (1, 0): np.arange(T),
             (1, 257): np.arange(T), (1, 514): np.arange(T)}
    ref = oracle.attention(q, k, v, causal=causal, rows=picks)
    got = {key: to_host(o[key[0], key[1]]) for key in picks}
    check_rows(got, ref, v, f"8-wave, B H = 1030, causal={causal}")


def test_attention_closed_forms():
    # Q = 0: uniform weights, the causal output is the prefix mean of V
    B, H, T = 1, 1, 300
    q = np.zeros((B, H, T, 128), np.uint16)
    _, k, v = qkv(B, H, T, seed=3)
    got = oracle.bf16_to_f32(run(q, k, v, True)[0, 0]).astype(np.float64)
    vf = oracle.bf16_to_f32(v[0, 0]).astype(np.float64)
    prefix = np.cumsum(vf, axis=0) / np.arange(1, T + 1)[:, None]
    assert np.abs(got - prefix).max() <= bf16_ulp(prefix).max() + 2.0 ** -8 * np.abs(vf).max()
    # row 0 under the causal mask is V[0] exactly (one weight of 1)
    assert np.array_equal(run(*qkv(1, 2, 77, seed=4), True)[:, :, 0], qkv(1, 2, 77, seed=4)[2][:, :, 0])


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_attention_bitwise_reproducible(dt):
    q, k, v = (to_dev(a) for a in qkv(2, 4, 700, seed=5, dt=dt))
    a = fk.attention_fwd(q, k, v)
    b = fk.attention_fwd(q, k, v)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_fp16_strided_and_closed_form():
    B, H, T, d = 2, 4, 300, 128
    rng = np.random.default_rng(17)
    base = [rng.standard_normal((B, T, H, d)).astype(np.float16) for _ in range(3)]
    qt, kt, vt = (to_dev(a).permute(0, 2, 1, 3) for a in base)
    ot = torch.empty((B, T, H, d), dtype=torch.float16, device=DEV).permute(0, 2, 1, 3)
    fk.fk_attention_fwd(qt, kt, vt, ot, causal=False)
    got = to_host(ot.contiguous())
    q, k, v = (np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in base)
    ref = oracle.attention(q, k, v, causal=False)
    rows = {(b, h): np.arange(T) for b in range(B) for h in range(H)}
    check_rows({key: got[key[0], key[1]] for key in rows},
               {key: ref[key[0], key[1]] for key in rows}, v, "fp16 B,T,H,d layout")
    # row 0 under the causal mask is V[0] exactly
    q, k, v = qkv(1, 2, 77, seed=4, dt="fp16")
    assert np.array_equal(run(q, k, v, True)[:, :, 0], v[:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_attention_wide_key_strides(causal):
    # K and V rows 2^25 + 8 elements apart: 64 rows of that stride pass 2^31
    # elements, so the kernel takes its 64-bit load-offset variant; T = 66 is
    # one whole 64-key block and a partial one (about 4.4 GB per operand)
    B, H, T, d = 1, 1, 66, 128
    stride = (1 << 25) + 8
    q, k, v = qkv(B, H, T, seed=23)
    span = (T - 1) * stride + d
    views = []
    for a in (k, v):
        buf = torch.empty(span, dtype=torch.bfloat16, device=DEV)
        view = buf.as_strided((B, H, T, d), (T * stride, T * stride, stride, 1))
        view.copy_(to_dev(a))
        views.append(view)
    o = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=DEV)
    fk.fk_attention_fwd(to_dev(q), views[0], views[1], o, causal=causal)
    got = to_host(o)
    ref = oracle.attention(q, k, v, causal=causal)
    check_rows({(0, 0): got[0, 0]}, {(0, 0): ref[0, 0]}, v, f"wide strides causal={causal}")
    del views
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_attention_wide_key_strides_eight_waves(causal):
    # The 64-bit load-offset variant in the 8-wave shape: every one of the
    # 2048 heads reads the same K and V rows, 2^25 + 8 elements apart (head
    # and batch strides 0), so 2048 workgroups (enough for 8 waves, full or
    # causal, on a 256-CU MI355X) fit in about 4.4 GB per operand; each head
    # has its own queries.
    B, H, T, d = 2, 1024, 66, 128
    stride = (1 << 25) + 8
    q, _, _ = qkv(B, H, T, seed=29)
    _, k1, v1 = qkv(1, 1, T, seed=30)
    span = (T - 1) * stride + d
    views = []
    for a in (k1, v1):
        buf = torch.empty(span, dtype=torch.bfloat16, device=DEV)
        one = buf.as_strided((1, 1, T, d), (0, 0, stride, 1))
        one.copy_(to_dev(a))
        views.append(buf.as_strided((B, H, T, d), (0, 0, stride, 1)))
    o = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=DEV)
    fk.fk_attention_fwd(to_dev(q), views[0], views[1], o, causal=causal)
    kb = np.broadcast_to(k1, (B, H, T, d))
    vb = np.broadcast_to(v1, (B, H, T, d))
    picks = {(0, 0): np.arange(T), (1, 1023): np.arange(T), (1, 77): np.arange(T)}
    ref = oracle.attention(q, kb, vb, causal=causal, rows=picks)
    got = {key: to_host(o[key[0], key[1]]) for key in picks}
    check_rows(got, ref, vb, f"wide strides, 8 waves, causal={causal}")
    del views
    torch.cuda.empty_cache()
