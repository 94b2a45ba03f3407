"""GPU parity of the prompt prefill (about 300 tokens for each of the two CFG
rows: "MiniMax Music 3, local"; TensorFold PR #987) against the oracle: the
row-wise RMSNorm (m3_rmsnorm_rows) and the dense GEMM on the matrix cores
(m3_prefill_gemm) with its epilogues, at sizes that span several tiles of
every tile shape (the 16 x 16 x 32 MFMA kernel's 64 x 128, 96 x 128 and 64 x
256, the 32 x 32 x 16 kernel's 128 x 128 and 128 x 256) with ragged M, N and K
step counts,
and at the full body shapes on sampled output columns the oracle computes
one row block at a time.  Every call goes
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import m3, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rand_w(N, K, seed):
    return synth.bits(synth.normal_bf16((N, K), seed, 0.02))


def rand_x(M, K, seed):
    return synth.bits(synth.activations(M, K, seed))


def gemm(W, a, epi=m3.EPI_NONE, out_f32=False, res=None, flags=0):
    N, K = W.shape
    pk = m3.pack(0, synth.from_bits(W, DEV), flags)
    y = m3.prefill_gemm(pk, N, K, synth.from_bits(a, DEV), epi=epi,
                        out_dtype=m3.OUT_F32 if out_f32 else m3.OUT_BF16,
                        residual=None if res is None else synth.from_bits(res, DEV))
    torch.cuda.synchronize()
    return y.cpu().numpy() if out_f32 else synth.bits(y)


# At 256 rows or more, 384 tiles of 128 x 256 select the 32 x 32 x 16
# kernel's 128 x 256 tiles ((1024, 12300): 392, the last 12 columns in a
# partial tile), else 192 tiles of 128 x 128 its 128 x 128 tiles ((1000,
# 4100), (1024, 4096) and (300, 8200)); then (600, 4096) and (650, 3000) reach the 96 x 128
# tiles (more than 256 tiles of 64 x 128, at most 256 of 96 x 128; 650 rows
# end in a partial tile); the others 64 x 128
@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (37, 200, 512), (600, 256, 512), (129, 130, 1024),
                                   (300, 520, 256), (37, 300, 8192), (1000, 4100, 128),
                                   (1024, 4096, 192), (600, 4096, 128), (650, 3000, 192),
                                   (1024, 12300, 64), (300, 8200, 192)])
def test_prefill_gemm_parity(M, N, K):
    W = rand_w(N, K, M + N)
    a = rand_x(M, K, K + 3)
    y_ex = O.gemv(O.Matrix(W, O.BF16), a)
    P.check_f32(gemm(W, a, out_f32=True), y_ex)
    P.check_bf16(gemm(W, a), y_ex)


@pytest.mark.parametrize("M,K,F,N", [(1, 512, 100, 200), (150, 512, 100, 200), (600, 512, 100, 200),
                                     (70, 8192, 100, 200), (1, 512, 99, 203), (150, 512, 99, 203),
                                     (600, 512, 99, 203), (70, 8192, 99, 203),
                                     (1000, 64, 2050, 4100), (1024, 64, 2051, 4099),
                                     (1024, 64, 6150, 12300), (1000, 192, 6151, 12301)])
def test_prefill_epilogues(M, K, F, N):
    """SwiGLU and residual epilogues; F = 100 / N = 200 give rows of whole
    16-byte chunks, F = 99 / N = 203 ragged tails and unaligned row strides;
    the last four run on the 32 x 32 x 16 kernel (the SwiGLU GEMM has N = 2F):
    128 x 128 tiles for N about 4100, 128 x 256 for N about 12300."""
    Wg, Wu = rand_w(F, K, 11), rand_w(F, K, 12)
    a = rand_x(M, K, 13)
    m = gemm(np.concatenate([Wg, Wu], 0), a, epi=m3.EPI_SWIGLU, flags=m3.PACK_GLU_INTERLEAVE)
    assert m.shape == (M, F)
    P.check_swiglu(m, O.gemv(O.Matrix(O.interleave_gate_up(Wg, Wu), O.BF16), a))
    W = rand_w(N, K, 14)
    h = rand_x(M, N, 15)
    y_ex = O.gemv(O.Matrix(W, O.BF16), a)
    P.check_residual(gemm(W, a, epi=m3.EPI_RESIDUAL, res=h), h, y_ex)
    # in place: the residual stream is the output
    hd = synth.from_bits(h, DEV)
    m3.prefill_gemm(m3.pack(0, synth.from_bits(W, DEV)), N, K, synth.from_bits(a, DEV), y=hd,
                    epi=m3.EPI_RESIDUAL, residual=hd)
    torch.cuda.synchronize()
    P.check_residual(synth.bits(hd), h, y_ex)


@pytest.mark.parametrize("M,K", [(1, 64), (600, 4096), (37, 2048)])
def test_rmsnorm_rows_parity(M, K):
    x = rand_x(M, K, 20 + M)
    g = synth.gamma_f32(K, 21).numpy()
    a = synth.bits(m3.rmsnorm_rows(synth.from_bits(x, DEV), torch.from_numpy(g).to(DEV), 1e-6))
    ref = O.rmsnorm(x, g, 1e-6)
    # one rounding of x r gamma: the fp32 r and two fp32 products may round a
    # value on the other side of a bf16 midpoint than the float64 oracle
    av, rv = O.bf16_to_f64(a), O.bf16_to_f64(ref)
    assert np.mean(a == ref) >= 0.99
    assert np.all(np.abs(av - rv) <= 2 * P.half_ulp(rv) + 1e-30)


@pytest.mark.parametrize("which", ["qkv", "o", "gate_up", "down"])
def test_prefill_full_size_sampled(which):
    """Full body shapes at M = 600: every output column of the first, a
    middle and the last row block of W checked against the oracle."""
    N, K, epi = {"qkv": (6144, 4096, m3.EPI_NONE), "o": (4096, 4096, m3.EPI_NONE),
                 "gate_up": (24576, 4096, m3.EPI_NONE), "down": (4096, 12288, m3.EPI_NONE)}[which]
    M = 600
    Wd = synth.normal_bf16((N, K), 30, 0.02, DEV)
    a = rand_x(M, K, 31)
    pk = m3.pack(0, Wd)
    y = m3.prefill_gemm(pk, N, K, synth.from_bits(a, DEV), out_dtype=m3.OUT_F32, epi=epi)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    W = synth.bits(Wd)
    M_ = O.Matrix(W, O.BF16)
    for r0 in (0, N // 2 + 16, N - 16):
        y_ex = O.gemv(M_, a, rows=(r0, 16))
        P.check_f32(y[:, r0:r0 + 16], y_ex)
