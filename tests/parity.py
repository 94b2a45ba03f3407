"""Comparison rules shared by the GPU parity tests (imported by tests only).

Tolerances (target: GEMV outputs within 1e-2 * rms(y) for bf16 out and
2e-3 * rms(y) for fp32 out; sampling bit-exact):

* fp32 out:  |y_gpu - y_exact| <= 2e-3 * rms(y_exact) per batch row.
* bf16 out:  the GPU value must be the bf16 rounding of a value within the
  fp32 bound, i.e. |y_gpu - y_exact| <= half_ulp_bf16(y) + 2e-3 * rms(y);
  and at least 99% of outputs equal the oracle's own bf16(y_exact).  (A bound
  of 1e-2 * rms against the unrounded value alone cannot hold: bf16's own
  half-ulp exceeds it once |y| > 2.56 rms.)
* epilogues that round intermediates (SwiGLU rounds gate and up, residual
  rounds the GEMV output) add half an ulp plus the fp32 bound of each rounded
  intermediate, propagated with the operation's derivative.
"""
from __future__ import annotations

import numpy as np

import oracle as O

REL = 2e-3


def half_ulp(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.frexp(v)[1]
    return np.ldexp(1.0, e - 9)


def row_rms(y):
    y = np.asarray(y, np.float64)
    return np.sqrt(np.mean(y * y, axis=-1, keepdims=True))


def check_f32(y_gpu, y_ex, rel=REL):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ex)
    bound = rel * row_rms(y_ex)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} fp32 outputs off; worst {np.max(err / bound):.3g}x bound"


def check_bf16(y_gpu_bits, y_ex, rel=REL, agree=0.99):
    y = O.bf16_to_f64(y_gpu_bits)
    err = np.abs(y - y_ex)
    bound = half_ulp(y_ex) * (1 + 1e-9) + rel * row_rms(y_ex)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} bf16 outputs off; worst {np.max(err / bound):.3g}x bound"
    same = np.mean(np.asarray(y_gpu_bits) == O.f64_to_bf16(y_ex))
    assert same >= agree, f"only {same:.4f} equal to the oracle's rounding"


def check_swiglu(m_gpu_bits, y_gu_ex, agree=0.98, rel=REL):
    """y_gu_ex: exact GEMV output over interleaved rows [B, 2F]."""
    g = y_gu_ex[:, 0::2]
    u = y_gu_ex[:, 1::2]
    dg = rel * row_rms(g) + half_ulp(g)
    du = rel * row_rms(u) + half_ulp(u)
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1 + g * (1 - sig)))
    m_ex = silu * u
    m = O.bf16_to_f64(m_gpu_bits)
    bound = (np.abs(u) * (dsilu * dg + 0.55 * dg * dg) + (np.abs(silu) + 1.1 * dg) * du
             + half_ulp(np.maximum(np.abs(m_ex), np.abs(m))) + 1e-6 * np.abs(m_ex) + 1e-30)
    err = np.abs(m - m_ex)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} SwiGLU outputs off; worst {np.max(err / bound):.3g}x"
    same = np.mean(np.asarray(m_gpu_bits) == O.swiglu_interleaved(y_gu_ex))
    assert same >= agree, f"only {same:.4f} equal to the oracle's SwiGLU"


def check_residual(h_gpu_bits, h_in_bits, y_ex, agree=0.98, rel=REL):
    h = O.bf16_to_f64(h_in_bits)
    ex = h + y_ex
    out = O.bf16_to_f64(h_gpu_bits)
    bound = (half_ulp(y_ex) + rel * row_rms(y_ex)
             + half_ulp(np.maximum(np.abs(ex), np.abs(out))) * (1 + 1e-9))
    err = np.abs(out - ex)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} residual outputs off; worst {np.max(err / bound):.3g}x"
    same = np.mean(np.asarray(h_gpu_bits) == O.residual(y_ex, h_in_bits))
    assert same >= agree, f"only {same:.4f} equal to the oracle's residual"


def classes(v):
    v = np.asarray(v, np.float64)
    return np.where(np.isnan(v), 3, np.where(np.isposinf(v), 1, np.where(np.isneginf(v), 2, 0)))


def unpack(packed: np.ndarray, fmt: int, N: int, K: int):
    """Decode the packed tile layout (include/m3.h) back to row-major arrays:
    bf16 -> uint16 [N, K]; int8 -> (q int8 [N, K], scales [N] or [N, K/128]);
    fp8-row -> (codes uint8 [N, K], scales [N])."""
    TK = 32 if fmt == O.BF16 else 64
    Kp = -(-K // TK) * TK
    T = Kp // TK
    nb = -(-N // 16)
    sb = {O.BF16: 0, O.I8ROW: 128, O.FP8ROW: 128, O.I8G128: -(-(K // 128) * 64 // 128) * 128}[fmt]
    bb = T * 1024 + sb
    blocks = np.ascontiguousarray(packed[: nb * bb]).reshape(nb, bb)
    tiles = np.ascontiguousarray(blocks[:, : T * 1024]).reshape(nb, T, 4, 16, 16)
    if fmt == O.BF16:
        w = tiles.view(np.uint16).reshape(nb, T, 4, 16, 8).transpose(0, 3, 1, 2, 4)
        return w.reshape(nb * 16, Kp)[:N, :K]
    q = tiles.view(np.uint8 if fmt == O.FP8ROW else np.int8).reshape(nb, T, 4, 16, 16)
    q = q.transpose(0, 3, 1, 2, 4).reshape(nb * 16, Kp)
    sc = np.ascontiguousarray(blocks[:, T * 1024:])
    if fmt in (O.I8ROW, O.FP8ROW):
        s = sc[:, :64].view(np.float32).reshape(nb * 16)
    else:
        G = K // 128
        s = sc[:, : G * 64].view(np.float32).reshape(nb * 16, G)
    return q[:N, :K], s[:N]


def check_bf16_vs_bf16(got_bits, want_bits, agree=0.99, rel=REL, width=None):
    """bf16 against the oracle's own bf16 result (rounded once from its float64
    value): per row of `width` values (the last axis by default),
    |got - want| <= 2 half-ulps of want (the oracle's rounding and ours) +
    rel * rms(row), which covers outputs that cancel towards zero, and at
    least `agree` of them identical (zeros of either sign equal)."""
    g = np.asarray(got_bits, np.uint16)
    w = np.asarray(want_bits, np.uint16)
    if width is not None:
        g, w = g.reshape(-1, width), w.reshape(-1, width)
    gv, wv = O.bf16_to_f64(g), O.bf16_to_f64(w)
    err = np.abs(gv - wv)
    bound = 2 * half_ulp(wv) * (1 + 1e-9) + rel * row_rms(wv)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} of {bad.size} bf16 outputs off; worst {np.max(err / bound):.3g}x bound"
    same = np.mean(gv == wv)
    assert same >= agree, f"only {same:.4f} equal to the oracle's rounding"
