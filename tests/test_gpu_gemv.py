"""GPU parity of the packer and the RMSNorm-fused GEMV family against the CPU
oracle (TensorFold PR #987 precision list: bf16, int8 per row, int8 per group
of 128; fused RMS norm; SwiGLU and residual epilogues; identity attention
stub), and of the fp8 (OCP E4M3, one scale per row) weight-only format.
Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import m3, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_dev(bits):
    return synth.from_bits(bits, DEV)


def rand_w(N, K, seed, std=0.02):
    return synth.bits(synth.normal_bf16((N, K), seed, std))


def rand_x(B, K, seed, std=1.0):
    return synth.bits(synth.activations(B, K, seed, std=std))


def rand_gamma(K, seed):
    return synth.gamma_f32(K, seed).numpy()


def run_gemv(fmt, W, x, gamma=None, out_f32=False, epi=m3.EPI_NONE, res=None, flags=0,
             stub=(0, 0), N=None, K=None):
    Wd = to_dev(W)
    pk = m3.pack(fmt, Wd, flags)
    N = W.shape[0] if N is None else N
    K = W.shape[1] if K is None else K
    xd = to_dev(x)
    gd = None if gamma is None else torch.from_numpy(gamma).to(DEV)
    rd = None if res is None else to_dev(res)
    y = m3.gemv(fmt, pk, N, K, xd, gamma=gd, eps=1e-6, stub_group=stub[0], stub_voff=stub[1],
                out_dtype=m3.OUT_F32 if out_f32 else m3.OUT_BF16, epi=epi, residual=rd)
    torch.cuda.synchronize()
    if out_f32:
        return y.cpu().numpy()
    return synth.bits(y)


def oracle_y(fmt, W, x, gamma=None):
    a = O.rmsnorm(x, gamma, 1e-6)
    return O.gemv(O.Matrix(W, fmt), a)


# ----------------------------------------------------------------- pack ---
@pytest.mark.parametrize("fmt,N,K", [(0, 37, 72), (1, 37, 80), (2, 37, 384), (0, 16, 4096),
                                     (1, 48, 4096), (2, 40, 2048), (3, 37, 80), (3, 48, 4096)])
def test_pack_bit_exact(fmt, N, K):
    W = rand_w(N, K, 1)
    W[3] = 0                                  # an all-zero row
    pk = m3.pack(fmt, to_dev(W)).cpu().numpy()
    assert pk.size == m3.packed_bytes(fmt, N, K)
    if fmt == 0:
        assert np.array_equal(P.unpack(pk, fmt, N, K), W)
    else:
        q, s = P.unpack(pk, fmt, N, K)
        qo, so = {1: O.quant_i8row, 2: O.quant_i8g128, 3: O.quant_fp8row}[fmt](W)
        assert np.array_equal(q, qo)
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32))


def test_pack_glu_interleave():
    F, K = 24, 64
    W = rand_w(2 * F, K, 2)
    pk = m3.pack(0, to_dev(W), m3.PACK_GLU_INTERLEAVE).cpu().numpy()
    got = P.unpack(pk, 0, 2 * F, K)
    assert np.array_equal(got, O.interleave_gate_up(W[:F], W[F:]))


# ------------------------------------------------------------ GEMV parity --
SHAPES = {0: (200, 520), 1: (200, 528), 2: (200, 640), 3: (200, 528)}   # several tiles, ragged N and K


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [1, 2, 3, 6, 8, 16, 33, 64])
def test_gemv_norm_parity(fmt, B):
    N, K = SHAPES[fmt]
    W = rand_w(N, K, 10 + fmt)
    x = rand_x(B, K, 20 + B)
    g = rand_gamma(K, 30)
    y_ex = oracle_y(fmt, W, x, g)
    P.check_bf16(run_gemv(fmt, W, x, g), y_ex)
    P.check_f32(run_gemv(fmt, W, x, g, out_f32=True), y_ex)


@pytest.mark.parametrize("fmt", [0, 2])
@pytest.mark.parametrize("B", [1, 2])
def test_gemv_norm_long_rows(fmt, B):
    """One or two normed rows of K = 8320 (more than one 8-value chunk per
    thread in the copy and in the normalising pass)."""
    N, K = 136, 8320
    W = rand_w(N, K, 15 + fmt)
    x = rand_x(B, K, 25 + B)
    g = rand_gamma(K, 35)
    y_ex = oracle_y(fmt, W, x, g)
    P.check_bf16(run_gemv(fmt, W, x, g), y_ex)
    P.check_f32(run_gemv(fmt, W, x, g, out_f32=True), y_ex)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("B,K", [(16, 5248), (11, 7296)])
def test_gemv_operand_from_memory(fmt, B, K):
    """Rows too long for LDS (B * K * 2 bytes over 160 KB): the 16-row MFMA
    kernel reads each batch's operand from memory next to its weights;
    ragged N, a partial 16-row tile at B = 11, plain, residual and SwiGLU
    outputs."""
    N = 136
    W = rand_w(N, K, 45 + fmt)
    x = rand_x(B, K, 55 + B)
    y_ex = oracle_y(fmt, W, x)
    P.check_f32(run_gemv(fmt, W, x, out_f32=True), y_ex)
    h = rand_x(B, N, 65 + B)
    P.check_residual(run_gemv(fmt, W, x, epi=m3.EPI_RESIDUAL, res=h), h, y_ex)
    F = 56
    Wg, Wu = rand_w(F, K, 75 + fmt), rand_w(F, K, 85 + fmt)
    m = run_gemv(fmt, np.concatenate([Wg, Wu], 0), x, epi=m3.EPI_SWIGLU,
                 flags=m3.PACK_GLU_INTERLEAVE)
    P.check_swiglu(m, oracle_y(fmt, O.interleave_gate_up(Wg, Wu), x))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [1, 6, 16])
def test_gemv_plain_and_residual(fmt, B):
    N, K = SHAPES[fmt]
    W = rand_w(N, K, 40 + fmt)
    x = rand_x(B, K, 50 + B)
    y_ex = oracle_y(fmt, W, x)
    P.check_f32(run_gemv(fmt, W, x, out_f32=True), y_ex)
    h = rand_x(B, N, 60 + B)
    P.check_residual(run_gemv(fmt, W, x, epi=m3.EPI_RESIDUAL, res=h), h, y_ex)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("B", [1, 6, 16])
def test_gemv_swiglu(fmt, B):
    F, K = 104, SHAPES[fmt][1]
    Wg, Wu = rand_w(F, K, 70 + fmt), rand_w(F, K, 80 + fmt)
    x = rand_x(B, K, 90 + B)
    g = rand_gamma(K, 31)
    stacked = np.concatenate([Wg, Wu], 0)
    m = run_gemv(fmt, stacked, x, g, epi=m3.EPI_SWIGLU, flags=m3.PACK_GLU_INTERLEAVE)
    y_gu = oracle_y(fmt, O.interleave_gate_up(Wg, Wu), x, g)
    assert m.shape == (B, F)
    P.check_swiglu(m, y_gu)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("B,group", [(1, 4), (6, 4), (16, 1)])
def test_gemv_attention_stub(fmt, B, group):
    n_heads, hd = 8, 128
    n_kv = n_heads // group
    nqkv = (n_heads + 2 * n_kv) * hd
    qkv = rand_x(B, nqkv, 100 + B)
    W = rand_w(256, n_heads * hd, 110 + fmt)
    voff = (n_heads + n_kv) * hd
    o = O.attn_stub(qkv, voff, n_heads, group, hd)
    y_ex = O.gemv(O.Matrix(W, fmt), o)
    h = rand_x(B, 256, 120)
    out = run_gemv(fmt, W, qkv, epi=m3.EPI_RESIDUAL, res=h, stub=(group, voff), K=n_heads * hd)
    P.check_residual(out, h, y_ex)


# ---------------------------------------------------- benchmark shapes -----
@pytest.mark.parametrize("out_f32", [False, True])
def test_single_rmsnorm_gemv_4096(out_f32):
    """RMSNorm + GEMV: x [1, 4096] ~ N(0,1), gamma 1 + N(0, 0.1), eps 1e-6,
    W [4096, 4096] ~ N(0, 0.02), seed 0."""
    W = synth.bits(synth.normal_bf16((4096, 4096), 2, 0.02))
    x = synth.bits(synth.normal_bf16((1, 4096), 0))
    g = synth.gamma_f32(4096, 1).numpy()
    y_ex = oracle_y(0, W, x, g)
    y = run_gemv(0, W, x, g, out_f32=out_f32)
    (P.check_f32 if out_f32 else P.check_bf16)(y, y_ex)


@pytest.mark.parametrize("fmt,B", [(0, 1), (0, 2), (1, 6), (0, 16)])
@pytest.mark.parametrize("which", ["qkv", "o", "down"])
def test_body_layer_shapes(fmt, B, which):
    """Qwen3-8B-shaped body matrices at the benchmark batch sizes."""
    N, K = {"qkv": (6144, 4096), "o": (4096, 4096), "down": (4096, 12288)}[which]
    W = synth.bits(synth.normal_bf16((N, K), 200 + fmt, 0.02, DEV))
    x = rand_x(B, K, 210 + B)
    g = None if which != "qkv" else rand_gamma(K, 32)
    P.check_f32(run_gemv(fmt, W, x, g, out_f32=True), oracle_y(fmt, W, x, g))


@pytest.mark.parametrize("fmt,B", [(0, 1), (1, 6), (0, 16)])
def test_body_gate_up_shape(fmt, B):
    F, K = 12288, 4096
    Wg = synth.bits(synth.normal_bf16((F, K), 300, 0.02, DEV))
    Wu = synth.bits(synth.normal_bf16((F, K), 301, 0.02, DEV))
    x = rand_x(B, K, 310)
    g = rand_gamma(K, 33)
    m = run_gemv(fmt, np.concatenate([Wg, Wu], 0), x, g, epi=m3.EPI_SWIGLU,
                 flags=m3.PACK_GLU_INTERLEAVE)
    P.check_swiglu(m, oracle_y(fmt, O.interleave_gate_up(Wg, Wu), x, g))


@pytest.mark.parametrize("which", ["qkv", "o", "gate_up", "down", "head"])
def test_depth_shapes_g128(which):
    """Depth decoder step matrices (hidden 2048, FFN 5632, 1024-row head), int8 g128, B = 6."""
    N, K = {"qkv": (6144, 2048), "o": (2048, 2048), "gate_up": (11264, 2048),
            "down": (2048, 5632), "head": (1024, 2048)}[which]
    W = synth.bits(synth.normal_bf16((N, K), 400, 0.02, DEV))
    x = rand_x(6, K, 410)
    g = rand_gamma(K, 34) if which in ("qkv", "gate_up", "head") else None
    P.check_f32(run_gemv(2, W, x, g, out_f32=True), oracle_y(2, W, x, g))


# ---------------------------------------------- determinism and classes ----
@pytest.mark.parametrize("fmt,B", [(0, 1), (1, 6), (2, 16), (3, 3)])
def test_repeat_byte_identical_and_rows_independent(fmt, B):
    N, K = SHAPES[fmt]
    W = rand_w(N, K, 500)
    x = rand_x(B, K, 510)
    g = rand_gamma(K, 35)
    a = run_gemv(fmt, W, x, g, out_f32=True)
    b = run_gemv(fmt, W, x, g, out_f32=True)
    assert a.tobytes() == b.tobytes()
    perm = np.random.default_rng(0).permutation(B)
    c = run_gemv(fmt, W, x[perm], g, out_f32=True)
    assert c.tobytes() == a[perm].tobytes()
    if B > 1:
        x2 = x.copy()
        x2[1:] = rand_x(B - 1, K, 520)
        d = run_gemv(fmt, W, x2, g, out_f32=True)
        assert d[0].tobytes() == a[0].tobytes()


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("norm", [False, True])
def test_nonfinite_classes(fmt, norm):
    """Non-finite outputs match the oracle's classes (TensorFold PR #987,
    "Kernel contract": non-finite outputs match their classes)."""
    N, K = SHAPES[fmt]
    W = rand_w(N, K, 600)
    W[5, :] = 0                                    # 0 * inf = NaN in that row
    x = rand_x(4, K, 610)
    x[0, 7] = 0x7F80                               # +inf
    x[1, 9] = 0xFF80                               # -inf
    x[2, 11] = 0x7FC0                              # NaN
    g = rand_gamma(K, 36) if norm else None
    y_ex = oracle_y(fmt, W, x, g)
    y = run_gemv(fmt, W, x, g, out_f32=True)
    assert np.array_equal(P.classes(y), P.classes(y_ex))
    fin = P.classes(y_ex) == 0
    assert np.allclose(y[3][fin[3]], y_ex[3][fin[3]], rtol=0, atol=2e-3 * P.row_rms(y_ex[3:4])[0, 0])
