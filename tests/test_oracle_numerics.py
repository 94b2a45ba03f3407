"""Pins of the CPU oracle's numeric building blocks against things other than
itself: exhaustive sweeps, exact rational arithmetic (fractions), closed forms
and library routines (torch).  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F


# ---------------------------------------------------------------- bf16 ----
def exact_bf16_of_fraction(x: Fraction) -> float:
    """Nearest bf16 (8 significant bits, ties to even) of an exact rational,
    found by brute force over the binade; normal range only."""
    if x == 0:
        return 0.0
    s = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): candidates k/128, k in [128, 256]
    k = int(a * 128)
    lo, hi = Fraction(k, 128), Fraction(k + 1, 128)
    if a - lo < hi - a:
        m = lo
    elif a - lo > hi - a:
        m = hi
    else:
        m = lo if k % 2 == 0 else hi
    return s * float(m * Fraction(2) ** e)


def test_bf16_roundtrip_exhaustive(oracle):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_to_f64(b)
    back = oracle.f64_to_bf16(v)
    nan = np.isnan(v)
    assert np.array_equal(back[~nan], b[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_matches_torch_rne_on_fp32(oracle):
    rng = np.random.default_rng(1)
    f = rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000)
    # add exact midpoints between neighbouring bf16 values (ties)
    b = rng.integers(0, 0x7F00, 20000).astype(np.uint32)
    mids = ((b << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, mids, -mids]).astype(np.float32)
    ours = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_from_f64_is_single_rounding(oracle):
    # doubles just above a bf16 midpoint whose fp32 rounding lands exactly on
    # the midpoint: one rounding goes up, a rounding through fp32 would tie.
    rng = np.random.default_rng(2)
    for _ in range(300):
        k = int(rng.integers(128, 256)) & ~1          # even significand below
        e = int(rng.integers(-20, 20))
        mid = Fraction(2 * k + 1, 256) * Fraction(2) ** e
        x = mid + Fraction(2) ** (e - 40)             # above the tie, below fp32 resolution
        got = oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([float(x)])))[0]
        assert got == exact_bf16_of_fraction(Fraction(float(x)))
        assert got > float(mid)


# ------------------------------------------------------------- RMSNorm ----
def _bf16(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows", [2, 4, 600])
def test_rmsnorm_vs_torch_float64(oracle, rows):
    """Served shapes of the Metal port's kernel contract (2, 4 and 600 rows of
    4096) against torch's RMS norm in float64: the oracle's output is the
    bf16 rounding of an fp32 value within three fp32 ulps of it (r rounded to
    fp32, two fp32 products), so it lies within half a bf16 ulp plus that,
    and it is the float64 value's own rounding except where that value sits
    within those ulps of a tie between two bf16 values."""
    g = torch.Generator().manual_seed(rows)
    x = torch.randn(rows, 4096, generator=g).to(torch.bfloat16)
    gam = (1 + 0.1 * torch.randn(4096, generator=g)).float()
    a = oracle.rmsnorm(_bf16(x), gam.numpy(), 1e-6)
    ref = F.rms_norm(x.double(), (4096,), gam.double(), eps=1e-6).numpy()
    av = oracle.bf16_to_f64(a)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    assert np.all(np.abs(av - ref) <= half_ulp * (1 + 1e-9) + 3 * 2.0 ** -24 * np.abs(ref))
    assert np.mean(a == oracle.f64_to_bf16(ref)) >= 0.999


@pytest.mark.parametrize("K", [64, 128, 4096, 12288])
def test_rmsnorm_steps_vs_torch_float32(oracle, K):
    """The norm's steps as torch library operations: r from a float64 sum of
    squares rounded to float32, then two float32 products and one bf16
    rounding: the oracle gives the same bits (an fp32 product fused or taken
    in another order would differ near bf16 ties)."""
    g = torch.Generator().manual_seed(K)
    x = (torch.randn(5, K, generator=g) * torch.tensor([1.0, 1e-3, 30.0, 0.5, 7.0])[:, None])
    x = x.to(torch.bfloat16)
    gam = (1 + 0.1 * torch.randn(K, generator=g)).float()
    r = (1.0 / torch.sqrt((x.double() ** 2).mean(1, keepdim=True) + 1e-6)).float()
    want = ((x.float() * r) * gam).to(torch.bfloat16)
    got = oracle.rmsnorm(_bf16(x), gam.numpy(), 1e-6)
    assert np.array_equal(got, _bf16(want))


def test_rmsnorm_constant_vector_closed_form(oracle):
    # x = c everywhere, eps = 0: r = 1/|c| so a = bf16(sign(c) * gamma) exactly
    gam = np.linspace(0.5, 1.5, 256).astype(np.float32)
    for c in [3.0, -0.375, 1e-3]:
        x = oracle.f64_to_bf16(np.full((1, 256), c))
        a = oracle.rmsnorm(x, gam, 0.0)
        expect = oracle.f32_to_bf16(np.sign(c) * gam)
        assert np.array_equal(a[0], expect)


def test_rmsnorm_scale_invariance_and_no_gamma(oracle):
    rng = np.random.default_rng(3)
    x = oracle.f64_to_bf16(rng.standard_normal((3, 512)))
    gam = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    x4 = oracle.f64_to_bf16(oracle.bf16_to_f64(x) * 4.0)   # exact power-of-two scale
    assert np.array_equal(oracle.rmsnorm(x, gam, 0.0), oracle.rmsnorm(x4, gam, 0.0))
    assert np.array_equal(oracle.rmsnorm(x, None, 1e-6), x)


def test_rmsnorm_nonfinite_classes(oracle):
    x = oracle.f64_to_bf16(np.ones((3, 64)))
    x[0, 5] = 0x7FC0   # NaN -> whole row NaN
    x[1, 7] = 0x7F80   # +inf -> r = 0: inf*0 = NaN at k=7, 0 elsewhere
    a = oracle.bf16_to_f64(oracle.rmsnorm(x, np.ones(64, np.float32), 1e-6))
    assert np.all(np.isnan(a[0]))
    assert np.isnan(a[1, 7]) and np.all(a[1, :7] == 0) and np.all(a[1, 8:] == 0)
    assert np.all(np.isfinite(a[2]))


# ---------------------------------------------------------- quantisers ----
def _fraction_quant(row_vals):
    amax = max(abs(Fraction(float(v))) for v in row_vals)
    s = np.float32(np.float32(float(amax)) / np.float32(127.0))   # IEEE fp32 division
    if s == 0:
        return [0] * len(row_vals), s
    q = []
    for v in row_vals:
        t = round(Fraction(float(v)) / Fraction(float(s)))       # ties to even
        q.append(max(-127, min(127, t)))
    return q, s


def test_quant_i8row_bruteforce_8x8(oracle):
    rng = np.random.default_rng(4)
    W = oracle.f64_to_bf16(rng.standard_normal((8, 8)) * 0.02)
    W[3] = 0                      # all-zero row
    q, s = oracle.quant_i8row(W)
    Wv = oracle.bf16_to_f64(W)
    for n in range(8):
        qq, ss = _fraction_quant(Wv[n])
        assert s[n] == ss and list(q[n]) == qq


def test_quant_i8g128_bruteforce(oracle):
    rng = np.random.default_rng(5)
    W = oracle.f64_to_bf16(rng.standard_normal((4, 256)) * 0.02)
    W[1, 128:] = 0                # zero group
    q, s = oracle.quant_i8g128(W)
    Wv = oracle.bf16_to_f64(W)
    for n in range(4):
        for g in range(2):
            qq, ss = _fraction_quant(Wv[n, g * 128:(g + 1) * 128])
            assert s[n, g] == ss and list(q[n, g * 128:(g + 1) * 128]) == qq


@pytest.mark.parametrize("fmt", [1, 2])
def test_quant_reconstruction_bounds(oracle, fmt):
    rng = np.random.default_rng(6 + fmt)
    W = oracle.f64_to_bf16(rng.standard_normal((64, 512)) * 0.02)
    if fmt == 1:
        q, s = oracle.quant_i8row(W)
        S = np.repeat(s[:, None], 512, 1).astype(np.float64)
        groups = q.reshape(64, 1, 512)
    else:
        q, s = oracle.quant_i8g128(W)
        S = np.repeat(s, 128, 1).astype(np.float64)
        groups = q.reshape(64, 4, 128)
    Wv = oracle.bf16_to_f64(W)
    assert np.all(np.abs(Wv - S * q) <= S / 2 * (1 + 1e-12))
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.abs(groups).max(-1) == 127)


# -------------------------------------------------------------- GEMVs -----
def _exact_dot(wrow, arow):
    return sum(Fraction(float(w)) * Fraction(float(a)) for w, a in zip(wrow, arow))


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_gemv_bruteforce_exact(oracle, fmt):
    rng = np.random.default_rng(10 + fmt)
    K = 8 if fmt != 2 else 256
    W = oracle.f64_to_bf16(rng.standard_normal((8, K)) * 0.02)
    a = oracle.f64_to_bf16(rng.standard_normal((3, K)))
    M = oracle.Matrix(W, fmt)
    y = oracle.gemv(M, a)
    av = oracle.bf16_to_f64(a)
    for n in range(8):
        if fmt == 0:
            wd = [Fraction(float(v)) for v in oracle.bf16_to_f64(W[n])]
        elif fmt == 1:
            wd = [Fraction(float(M.s[n])) * int(v) for v in M.q[n]]
        else:
            wd = [Fraction(float(M.s[n, k // 128])) * int(M.q[n, k]) for k in range(K)]
        for b in range(3):
            ex = sum(w * Fraction(float(x)) for w, x in zip(wd, av[b]))
            assert abs(float(ex) - y[b, n]) <= 1e-13 * max(1.0, abs(float(ex)))


def test_gemv_identity(oracle):
    K = 64
    eye = oracle.f64_to_bf16(np.eye(K))
    rng = np.random.default_rng(12)
    a = oracle.f64_to_bf16(rng.standard_normal((2, K)))
    y = oracle.gemv(oracle.Matrix(eye, 0), a)
    assert np.array_equal(y, oracle.bf16_to_f64(a))
    y_rows = oracle.gemv(oracle.Matrix(eye, 0), a, rows=(10, 5))
    assert np.array_equal(y_rows, oracle.bf16_to_f64(a)[:, 10:15])


# ---------------------------------------------------------- epilogues -----
def test_swiglu_vs_torch_silu(oracle):
    rng = np.random.default_rng(13)
    y = rng.standard_normal((2, 2 * 300)) * 3
    y[0, 0] = 0.0                       # silu(0) = 0
    m = oracle.bf16_to_f64(oracle.swiglu_interleaved(y))
    g = oracle.bf16_to_f64(oracle.f64_to_bf16(y[:, 0::2]))
    u = oracle.bf16_to_f64(oracle.f64_to_bf16(y[:, 1::2]))
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    assert np.all(np.abs(m - ref) <= half_ulp * (1 + 1e-9) + 1e-300)
    assert m[0, 0] == 0.0
    big = oracle.bf16_to_f64(oracle.swiglu_interleaved(np.array([[40.0, 1.5]])))
    assert big[0, 0] == 60.0            # silu(40) = 40 to far below bf16 resolution


def test_residual_exact_small_integers(oracle):
    y = np.array([1.0, -3.0, 0.5, 1e-3])
    h = oracle.f64_to_bf16(np.array([2.0, 3.0, 0.25, 256.0]))
    out = oracle.bf16_to_f64(oracle.residual(y, h))
    assert list(out[:3]) == [3.0, 0.0, 0.75]
    assert out[3] == 256.0              # 256 + 1e-3 rounds back to 256 in bf16


def test_attn_stub_is_one_key_softmax_attention(oracle):
    """With a single cached position, softmax attention returns the value
    head of each query head's KV group (torch's SDPA as the library routine)."""
    rng = np.random.default_rng(14)
    B, nh, nkv, hd = 2, 8, 2, 16
    qkv = oracle.f64_to_bf16(rng.standard_normal((B, (nh + 2 * nkv) * hd)))
    o = oracle.attn_stub(qkv, voff=(nh + nkv) * hd, n_heads=nh, group=nh // nkv, hd=hd)
    v = torch.from_numpy(oracle.bf16_to_f64(qkv))
    q = v[:, :nh * hd].reshape(B, nh, 1, hd)
    k = v[:, nh * hd:(nh + nkv) * hd].reshape(B, nkv, 1, hd).repeat_interleave(nh // nkv, 1)
    vv = v[:, (nh + nkv) * hd:].reshape(B, nkv, 1, hd).repeat_interleave(nh // nkv, 1)
    ref = F.scaled_dot_product_attention(q, k, vv).reshape(B, nh * hd).numpy()
    assert np.array_equal(oracle.bf16_to_f64(o), ref)
