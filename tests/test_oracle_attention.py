"""Pins of the oracle's decode attention: the RoPE table, per-head q/k RMSNorm
+ RoPE with the KV-cache writes, and softmax attention over the cached
positions ("MiniMax Music 3, local" and TensorFold PR #987, kernel list: per-
head q/k norm and RoPE, decode attention over the cached keys, the depth
decoder's attention over the codebook positions; Qwen3's RoPE base 1e6).

Pinned by closed forms (position 0, frequency 0, one-hot heads whose rotation
is cos/sin of the position, a two-key softmax), invariants (rotation keeps
pair norms; dot products depend only on the position difference), the
identity-attention special case T = 1, GQA head mapping, masking of positions
past T, and torch's scaled_dot_product_attention in float64 as an independent
library routine.  CPU only."""
import math

import numpy as np
import pytest
import torch

HD = 128


def bf16(x):
    """float64 -> bf16 bits by torch's cast (through fp32)."""
    t = torch.as_tensor(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulps_apart(a, b):
    a = np.asarray(a, np.uint16).astype(np.int32)
    b = np.asarray(b, np.uint16).astype(np.int32)
    # bf16 bits are sign-magnitude; map to a monotone integer line
    ma = np.where(a & 0x8000, -(a & 0x7FFF), a)
    mb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ma - mb)


def cache(B, n_kv, max_pos):
    return np.zeros((B, n_kv, max_pos, HD), np.uint16)


def test_rope_table_closed_forms(oracle):
    t = oracle.rope_table(2001).astype(np.float64)
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)
    # pair 0 turns by one radian per position
    for p in (1, 7, 1000, 2000):
        assert t[p, 0, 0] == np.float32(math.cos(p)) and t[p, 0, 1] == np.float32(math.sin(p))
    # pair 32 turns by theta^-1/2 = 1e-3 rad per position: position 1000 is one radian
    assert abs(t[1000, 32, 0] - math.cos(1.0)) < 1e-7 and abs(t[1000, 32, 1] - math.sin(1.0)) < 1e-7
    # the angle per position recovered from position 1 is theta^(-i/64), geometric in i
    ang = np.arctan2(t[1, :, 1], t[1, :, 0])
    assert np.allclose(ang, 1e6 ** (-np.arange(64) / 64.0), rtol=2e-7, atol=1e-12)
    assert np.allclose(t[..., 0] ** 2 + t[..., 1] ** 2, 1.0, atol=3e-7)


def _qkv(B, n_q, n_kv, seed):
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal((B, (n_q + 2 * n_kv) * HD)) * 1.5)


def test_position_zero_is_the_head_rmsnorm(oracle):
    """At position 0 the rotation is the identity: q and k are the per-head
    RMSNorm of their heads, bf16(x r gamma) with r over the head's 128 values;
    v is copied unchanged into the cache."""
    B, n_q, n_kv, eps = 3, 4, 2, 1e-6
    rng = np.random.default_rng(1)
    qkv = _qkv(B, n_q, n_kv, 2)
    qg = (1.0 + 0.1 * rng.standard_normal(HD)).astype(np.float32)
    kg = (1.0 + 0.1 * rng.standard_normal(HD)).astype(np.float32)
    kc, vc = cache(B, n_kv, 5), cache(B, n_kv, 5)
    q = oracle.qk_norm_rope(qkv, n_q, n_kv, qg, kg, eps, oracle.rope_table(5), 0, kc, vc)
    x = f64(qkv).reshape(B, n_q + 2 * n_kv, HD)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=2, keepdims=True) + eps)
    want_q = bf16(x[:, :n_q] * r[:, :n_q] * qg.astype(np.float64)).reshape(B, -1)
    want_k = bf16(x[:, n_q:n_q + n_kv] * r[:, n_q:n_q + n_kv] * kg.astype(np.float64))
    for got, want in ((q, want_q), (kc[:, :, 0], want_k)):
        assert np.mean(got == want) >= 0.999 and ulps_apart(got, want).max() <= 1
    assert np.array_equal(vc[:, :, 0], qkv.reshape(B, n_q + 2 * n_kv, HD)[:, n_q + n_kv:])
    assert not kc[:, :, 1:].any() and not vc[:, :, 1:].any()


@pytest.mark.parametrize("pos", [1, 5, 999])
def test_one_hot_head_turns_into_its_partner(oracle, pos):
    """A head whose only nonzero value is element 0 normalises to
    x'_0 = sqrt(128) gamma_0; the rotation sends it to y_0 = x'_0 cos(pos),
    y_64 = x'_0 sin(pos) (pair i with i + 64, angle pos for pair 0) and leaves
    the rest zero."""
    n_q, n_kv = 1, 1
    qkv = np.zeros((1, 3 * HD), np.uint16)
    qkv[0, 0] = bf16(0.75)[()]
    qkv[0, HD] = bf16(-2.0)[()]
    g = np.full(HD, 1.25, np.float32)
    kc, vc = cache(1, 1, pos + 1), cache(1, 1, pos + 1)
    q = oracle.qk_norm_rope(qkv, n_q, n_kv, g, g, 0.0, oracle.rope_table(pos + 1), pos, kc, vc)
    c, s = np.float32(math.cos(pos)), np.float32(math.sin(pos))
    for sign, y in ((1.0, q[0]), (-1.0, kc[0, 0, pos])):
        x0 = f64(bf16(sign * math.sqrt(128) * 1.25))[()]
        assert y[0] == bf16(x0 * float(c))[()] and y[64] == bf16(x0 * float(s))[()]
        assert np.all(f64(np.delete(y, [0, 64])) == 0.0)     # zeros (of either sign)


def test_rotation_keeps_pair_norms_and_relative_positions(oracle):
    B, n_q, n_kv = 2, 2, 1
    rng = np.random.default_rng(3)
    qkv = _qkv(B, n_q, n_kv, 4)
    g = (1.0 + 0.1 * rng.standard_normal(HD)).astype(np.float32)
    tab = oracle.rope_table(600)

    def rot(pos):
        kc, vc = cache(B, n_kv, 600), cache(B, n_kv, 600)
        q = oracle.qk_norm_rope(qkv, n_q, n_kv, g, g, 1e-6, tab, pos, kc, vc)
        return f64(q).reshape(B, n_q, HD), f64(kc[:, :, pos])

    q0, k0 = rot(0)
    for pos in (3, 250, 599):
        q, k = rot(pos)
        n0 = q0[..., :64] ** 2 + q0[..., 64:] ** 2
        n1 = q[..., :64] ** 2 + q[..., 64:] ** 2
        assert np.all(np.abs(n1 - n0) <= 2 ** -6 * n0 + 1e-30)
    # q at position m against k at position n depends on m - n only
    for (m, n), (m2, n2) in (((10, 3), (207, 200)), ((599, 0), (599, 0)), ((40, 90), (540, 590))):
        qa, _ = rot(m)
        _, ka = rot(n)
        qb, _ = rot(m2)
        _, kb = rot(n2)
        da = np.einsum("bhd,bd->bh", qa, ka[:, 0])
        db = np.einsum("bhd,bd->bh", qb, kb[:, 0])
        scale = np.linalg.norm(qa, axis=2) * np.linalg.norm(ka[:, 0], axis=1)[:, None]
        assert np.all(np.abs(da - db) <= 2e-2 * scale)
    # the rotation is not trivial: moving k alone changes the dot products
    assert np.any(np.abs(np.einsum("bhd,bd->bh", rot(7)[0], rot(0)[1][:, 0])
                         - np.einsum("bhd,bd->bh", rot(0)[0], rot(7)[1][:, 0])) > 1e-3)


def _kv(B, n_kv, max_pos, T, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    kc, vc = cache(B, n_kv, max_pos), cache(B, n_kv, max_pos)
    kc[:, :, :T] = bf16(rng.standard_normal((B, n_kv, T, HD)) * scale)
    vc[:, :, :T] = bf16(rng.standard_normal((B, n_kv, T, HD)))
    return kc, vc


def test_one_position_is_the_identity_stub(oracle):
    """T = 1: softmax over one key is 1, so every q head reads its KV group's v."""
    B, n_q, n_kv = 3, 8, 2
    kc, vc = _kv(B, n_kv, 4, 1, 5)
    q = bf16(np.random.default_rng(6).standard_normal((B, n_q * HD)))
    out = oracle.decode_attention(q, kc, vc, 1, n_q, n_kv).reshape(B, n_q, HD)
    for h in range(n_q):
        assert np.array_equal(out[:, h], vc[:, h // (n_q // n_kv), 0])


def test_equal_keys_average_the_values_and_gqa_groups(oracle):
    B, n_q, n_kv, T = 2, 8, 2, 9
    kc, vc = _kv(B, n_kv, 12, T, 7)
    kc[:, :, :T] = kc[:, :, :1]                       # every key the same
    q = bf16(np.random.default_rng(8).standard_normal((B, n_q * HD)))
    out = oracle.decode_attention(q, kc, vc, T, n_q, n_kv).reshape(B, n_q, HD)
    mean = f64(vc[:, :, :T]).mean(axis=2)
    for h in range(n_q):
        want = bf16(mean[:, h // 4])
        assert np.mean(out[:, h] == want) >= 0.99 and ulps_apart(out[:, h], want).max() <= 1
    # values constant per KV head: each q head returns its group's constant
    vc[:, :, :T] = bf16(np.arange(1, n_kv + 1, dtype=np.float64)[None, :, None, None]
                        * np.ones((B, n_kv, T, HD)))
    kc2, _ = _kv(B, n_kv, 12, T, 9)
    out = oracle.decode_attention(q, kc2, vc, T, n_q, n_kv).reshape(B, n_q, HD)
    for h in range(n_q):
        assert np.all(f64(out[:, h]) == h // 4 + 1)


def test_two_keys_closed_form_fixes_the_scale(oracle):
    """k_0 - k_1 along q gives p_0 = 1 / (1 + exp(-(s_0 - s_1) / sqrt(128)));
    with v_0 = 1 and v_1 = 0 the output is p_0."""
    q = np.zeros((1, HD), np.float64)
    q[0, :4] = 1.0
    kc, vc = cache(1, 1, 2), cache(1, 1, 2)
    kc[0, 0, 0, :4] = bf16(2.0)[()]                  # s_0 = 8
    kc[0, 0, 1, :4] = bf16(-1.0)[()]                 # s_1 = -4
    vc[0, 0, 0] = bf16(1.0)[()]
    out = oracle.decode_attention(bf16(q), kc, vc, 2, 1, 1)
    p0 = 1.0 / (1.0 + math.exp(-12.0 / math.sqrt(128.0)))
    assert np.all(out[0] == bf16(p0)[()])


def test_positions_past_T_take_no_part(oracle):
    B, n_q, n_kv, T = 2, 4, 1, 6
    kc, vc = _kv(B, n_kv, 10, T, 10)
    q = bf16(np.random.default_rng(11).standard_normal((B, n_q * HD)))
    ref = oracle.decode_attention(q, kc, vc, T, n_q, n_kv)
    kc[:, :, T:] = bf16(1e30)[()]
    vc[:, :, T:] = 0x7FC0                             # NaN
    assert np.array_equal(oracle.decode_attention(q, kc, vc, T, n_q, n_kv), ref)


@pytest.mark.parametrize("T", [2, 37, 300])
def test_matches_torch_sdpa_float64(oracle, T):
    B, n_q, n_kv = 2, 8, 2
    kc, vc = _kv(B, n_kv, T + 3, T, 12 + T, scale=0.5)
    q = bf16(np.random.default_rng(13).standard_normal((B, n_q * HD)))
    out = oracle.decode_attention(q, kc, vc, T, n_q, n_kv)
    qt = torch.from_numpy(f64(q).reshape(B, n_q, 1, HD))
    kt = torch.from_numpy(f64(kc[:, :, :T])).repeat_interleave(n_q // n_kv, dim=1)
    vt = torch.from_numpy(f64(vc[:, :, :T])).repeat_interleave(n_q // n_kv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()
    want = bf16(ref.reshape(B, n_q * HD))
    assert np.mean(out == want) >= 0.99 and ulps_apart(out, want).max() <= 1


def _small_model(seed=3):
    from autoregressive_audio_lm_amd import configs, synth
    cfg = configs.config("frame-small")
    md = synth.model_to_numpy(synth.make_model(cfg, configs.BF16, configs.BF16, configs.I8G128,
                                               seed=seed))
    return cfg, md, synth


def test_frame_at_position_zero_has_the_stub_body(oracle):
    """Attention over one cached position is the identity stub: the first
    frame at position 0 has the stub frame's body output, semantic code and
    first depth code (the depth step 1 also attends over one position)."""
    cfg, md, synth = _small_model()
    x = synth.bits(synth.activations(3, cfg["H"], seed=6))
    stub = oracle.OracleModel(md)
    att = oracle.OracleModel(md, attention=1, max_pos=16, pos0=0)
    c_s, x_s, t_s = oracle.decode_frame(stub, x, seed=8, frame=0, trace=True)
    c_a, x_a, t_a = oracle.decode_frame(att, x, seed=8, frame=0, trace=True)
    assert np.array_equal(t_s["h_body"], t_a["h_body"])
    assert np.array_equal(c_s[:, :2], c_a[:, :2])


def test_frames_fill_the_cache_at_their_positions(oracle):
    """Frame f writes k and v at body position pos0 + f of every layer; later
    frames read the earlier positions (so their body output changes)."""
    cfg, md, synth = _small_model()
    x = synth.bits(synth.activations(2, cfg["H"], seed=7))
    att = oracle.OracleModel(md, attention=1, max_pos=16, pos0=4)
    stub = oracle.OracleModel(md)
    for f in range(3):
        _, _, ta = oracle.decode_frame(att, x, seed=1, frame=f, trace=True)
        _, _, ts = oracle.decode_frame(stub, x, seed=1, frame=f, trace=True)
        # position 4 + f attends over 5 + f positions (the prompt's, zero here, and the
        # frames' own), so the body differs from the stub's
        assert not np.array_equal(ta["h_body"], ts["h_body"])
    for kc, vc in zip(att.kcache, att.vcache):
        filled = np.any(kc != 0, axis=(0, 1, 3))
        assert filled.tolist() == [p in (4, 5, 6) for p in range(16)]
        assert np.array_equal(np.any(vc != 0, axis=(0, 1, 3)), filled)
    # the depth caches hold the 7 codebook positions of the last frame
    for dk in att.dkcache:
        assert np.any(dk != 0, axis=(0, 1, 3)).tolist() == [True] * 7 + [False]
