"""Pins of the oracle's fp8 weight-only format (OCP FP8 E4M3: bias 7, no
infinity, largest finite 448; one fp32 scale per row, absmax / 448).  The
pages list fp8 weight-only only as a result on another stack (diffusers
issue #14486 and MiniMax-Music3 issue #2, negative results), so the format
is the reading taken here.

Pinned by: torch's float8_e4m3fn as a library routine (every code decoded,
float32 values encoded), round trips and tie-to-even midpoints from the
definition, saturation, the quantiser's reconstruction bound and its
largest code per row, and exact rational brute force of the GEMV.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch


def test_decode_every_code_matches_torch(oracle):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2      # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(0x01) == 2.0 ** -9


def test_encode_round_trip_and_ties_to_even(oracle):
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for c in finite:
        assert oracle.fp8_encode(oracle.fp8_decode(c)) == c
    # midpoints between neighbouring positive values go to the even mantissa
    pos = sorted({oracle.fp8_decode(c) for c in range(0x7F)})
    for lo, hi in zip(pos, pos[1:]):
        c = oracle.fp8_encode((lo + hi) / 2)
        want = oracle.fp8_encode(lo) if oracle.fp8_encode(lo) % 2 == 0 else oracle.fp8_encode(hi)
        assert c == want, (lo, hi)
    # saturation (no infinity in the format) and NaN
    assert oracle.fp8_encode(448.0) == 0x7E and oracle.fp8_encode(463.9) == 0x7E
    assert oracle.fp8_encode(1e30) == 0x7E and oracle.fp8_encode(-1e30) == 0xFE
    assert oracle.fp8_encode(float("nan")) == 0x7F


def test_encode_matches_torch_on_float32_values(oracle):
    rng = np.random.default_rng(70)
    v = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(20000) * 0.01,
                        rng.uniform(-447, 447, 20000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_quant_fp8row_bounds(oracle):
    rng = np.random.default_rng(71)
    W = oracle.f64_to_bf16(rng.standard_normal((64, 512)) * 0.02)
    W[5] = 0                                               # all-zero row
    q, s = oracle.quant_fp8row(W)
    Wv = oracle.bf16_to_f64(W)
    amax = np.abs(Wv).max(1)
    assert s[5] == 0 and np.all(q[5] == 0)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    dec = np.vectorize(oracle.fp8_decode)(q)
    S = s[:, None].astype(np.float64)
    # |W - s dec(q)| <= half the spacing of E4M3 at dec(q), in units of s
    t = np.abs(Wv / np.where(S == 0, 1, S))
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    half = 2.0 ** (e - 4)
    nz = S[:, 0] > 0
    assert np.all(np.abs(t[nz] - np.abs(dec[nz])) <= half[nz] * (1 + 1e-12) + 1e-300)
    assert np.all(np.abs(dec[nz]).max(1) == 448.0)        # the row's absmax maps to 448
    assert np.all(np.sign(dec[nz]) * np.sign(Wv[nz]) >= 0)


def test_gemv_fp8row_bruteforce_exact(oracle):
    rng = np.random.default_rng(72)
    W = oracle.f64_to_bf16(rng.standard_normal((8, 16)) * 0.02)
    a = oracle.f64_to_bf16(rng.standard_normal((3, 16)))
    M = oracle.Matrix(W, oracle.FP8ROW)
    y = oracle.gemv(M, a)
    av = oracle.bf16_to_f64(a)
    dec = torch.from_numpy(M.q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for n in range(8):
        wd = [Fraction(float(M.s[n])) * Fraction(float(d)) for d in dec[n]]
        for b in range(3):
            ex = sum(w * Fraction(float(x)) for w, x in zip(wd, av[b]))
            assert abs(float(ex) - y[b, n]) <= 1e-13 * max(1.0, abs(float(ex)))


def test_matrix_bytes_fp8row(oracle):
    assert oracle.matrix_bytes(oracle.FP8ROW, 6144, 4096) == 6144 * 4096 + 4 * 6144
