"""GPU parity of decode attention against the oracle ("MiniMax Music 3,
local" and TensorFold PR #987's kernel list: per-head q/k norm + RoPE, decode
attention over the cached keys with split keys and a merge, the depth
decoder's attention over its codebook positions): the RoPE table, the q/k
norm + RoPE with its cache writes, and the attention at the body's 32:8 heads,
the depth decoder's 16:16 and the other supported groupings, from one cached
position to 1800 (60 s of frames plus a prompt), across the one-chunk and
split-and-merge paths.  Both sides build their own RoPE tables and caches;
every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import m3, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
HD = 128


def rnd_bf16(shape, seed, std=1.0):
    return synth.bits(synth.normal_bf16(shape, seed, std))


def dev(bits):
    return synth.from_bits(np.ascontiguousarray(bits), DEV)


def test_rope_table_matches_the_oracle():
    got = m3.rope_table(4096).cpu().numpy()
    want = O.rope_table(4096)
    gi, wi = got.view(np.int32), want.view(np.int32)
    assert np.abs(gi - wi).max() <= 1                  # float64 trig on both sides
    assert np.mean(gi == wi) >= 0.9999


@pytest.mark.parametrize("n_q,n_kv,B,pos", [(32, 8, 3, 0), (32, 8, 2, 7), (32, 8, 1, 1799),
                                            (16, 16, 4, 6), (8, 4, 2, 300)])
def test_qk_norm_rope_and_cache_writes(n_q, n_kv, B, pos):
    max_pos = pos + 3
    ldqkv = (n_q + 2 * n_kv) * HD + 64                # a padded row stride
    qkv = rnd_bf16((B, ldqkv), 100 + pos, 1.5)
    qg = (1.0 + 0.1 * np.random.default_rng(1).standard_normal(HD)).astype(np.float32)
    kg = (1.0 + 0.1 * np.random.default_rng(2).standard_normal(HD)).astype(np.float32)
    kc, vc = m3.kv_cache(B, n_kv, max_pos)
    q = m3.qk_norm_rope(dev(qkv), n_q, n_kv, torch.from_numpy(qg).to(DEV),
                        torch.from_numpy(kg).to(DEV), m3.rope_table(max_pos), pos, kc, vc)
    torch.cuda.synchronize()
    okc = np.zeros((B, n_kv, max_pos, HD), np.uint16)
    ovc = np.zeros_like(okc)
    oq = O.qk_norm_rope(qkv, n_q, n_kv, qg, kg, 1e-6, O.rope_table(max_pos), pos, okc, ovc)
    P.check_bf16_vs_bf16(synth.bits(q), oq, width=HD)
    gk, gv = synth.bits(kc), synth.bits(vc)
    P.check_bf16_vs_bf16(gk[:, :, pos], okc[:, :, pos], width=HD)
    assert np.array_equal(gv, ovc)                     # v copied bit for bit; nothing else written
    others = np.delete(gk, pos, axis=2)
    assert not others.any()


def fill_cache(B, n_kv, max_pos, T, seed, kscale):
    kc = np.zeros((B, n_kv, max_pos, HD), np.uint16)
    vc = np.zeros_like(kc)
    kc[:, :, :T] = rnd_bf16((B, n_kv, T, HD), seed, kscale)
    vc[:, :, :T] = rnd_bf16((B, n_kv, T, HD), seed + 1)
    return kc, vc


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (16, 16), (8, 4), (16, 2)])
@pytest.mark.parametrize("T", [1, 2, 8, 37, 128, 129, 300])
def test_attention_parity(n_q, n_kv, T):
    B, max_pos = 3, T + 5
    kc, vc = fill_cache(B, n_kv, max_pos, T, 10 * T + n_kv, 3.0)
    # positions past T hold values that would show if read
    kc[:, :, T:] = 0x7F00
    vc[:, :, T:] = 0x7FC0
    q = rnd_bf16((B, n_q * HD), T + 7)
    got = m3.decode_attention(dev(q), n_q, n_kv, dev(kc), dev(vc), T)
    torch.cuda.synchronize()
    want = O.decode_attention(q, kc, vc, T, n_q, n_kv)
    P.check_bf16_vs_bf16(synth.bits(got), want, width=HD)


def test_attention_full_size_body():
    """The body at 16 rows (8 songs) and 1800 cached positions: 15 chunks
    merged; checked in full against the oracle."""
    B, n_q, n_kv, T = 16, 32, 8, 1800
    kc, vc = fill_cache(B, n_kv, T, T, 77, 2.0)
    q = rnd_bf16((B, n_q * HD), 78)
    got = m3.decode_attention(dev(q), n_q, n_kv, dev(kc), dev(vc), T)
    torch.cuda.synchronize()
    P.check_bf16_vs_bf16(synth.bits(got), O.decode_attention(q, kc, vc, T, n_q, n_kv), width=HD)


def test_strides_and_workspace_reuse():
    B, n_q, n_kv, T = 2, 32, 8, 300
    kc, vc = fill_cache(B, n_kv, 512, T, 5, 2.0)
    q = rnd_bf16((B, n_q * HD + 128), 6)
    ws = m3.attention_workspace(B, n_q, n_kv, T)
    out = torch.zeros(B, n_q * HD + 64, dtype=torch.bfloat16, device=DEV)
    kd, vd, qd = dev(kc), dev(vc), dev(q)
    for T_ in (T, 129, 40):
        m3.decode_attention(qd[:, :n_q * HD], n_q, n_kv, kd, vd, T_, out=out[:, :n_q * HD],
                            workspace=ws)
        torch.cuda.synchronize()
        want = O.decode_attention(q[:, :n_q * HD], kc, vc, T_, n_q, n_kv)
        P.check_bf16_vs_bf16(synth.bits(out[:, :n_q * HD]), want, width=HD)
        assert not synth.bits(out[:, n_q * HD:]).any()


def test_decode_steps_build_the_cache():
    """Twenty decode steps: each step's QKV row goes through the norm + RoPE
    at its position into the cache, then attention over the positions so far;
    both sides keep their own caches."""
    B, n_q, n_kv, steps = 2, 32, 8, 20
    ldqkv = (n_q + 2 * n_kv) * HD
    qg = (1.0 + 0.1 * np.random.default_rng(3).standard_normal(HD)).astype(np.float32)
    kg = (1.0 + 0.1 * np.random.default_rng(4).standard_normal(HD)).astype(np.float32)
    qgd, kgd = torch.from_numpy(qg).to(DEV), torch.from_numpy(kg).to(DEV)
    rope, orope = m3.rope_table(steps), O.rope_table(steps)
    kc, vc = m3.kv_cache(B, n_kv, steps)
    okc = np.zeros((B, n_kv, steps, HD), np.uint16)
    ovc = np.zeros_like(okc)
    for pos in range(steps):
        qkv = rnd_bf16((B, ldqkv), 500 + pos, 1.5)
        q = m3.qk_norm_rope(dev(qkv), n_q, n_kv, qgd, kgd, rope, pos, kc, vc)
        o = m3.decode_attention(q, n_q, n_kv, kc, vc, pos + 1)
        torch.cuda.synchronize()
        oq = O.qk_norm_rope(qkv, n_q, n_kv, qg, kg, 1e-6, orope, pos, okc, ovc)
        # the oracle attends from its own q and cache; both agree to a bf16 ulp
        # at every step (the caches themselves are compared too)
        P.check_bf16_vs_bf16(synth.bits(kc[:, :, :pos + 1]), okc[:, :, :pos + 1], width=HD)
        P.check_bf16_vs_bf16(synth.bits(o), O.decode_attention(oq, okc, ovc, pos + 1, n_q, n_kv),
                             agree=0.97, rel=1e-2, width=HD)


@pytest.mark.parametrize("B,n_q,n_kv", [(2, 32, 8), (1, 16, 16), (5, 8, 4)])
def test_decode_attention_step_equals_the_two_calls(B, n_q, n_kv):
    """m3_decode_attention_step (one launch plus the merge) gives the bytes
    of m3_qk_norm_rope followed by m3_decode_attention: the output and both
    caches, at positions with one chunk and with several (over seeded
    earlier positions)."""
    max_pos = 400
    ldqkv = (n_q + 2 * n_kv) * HD
    qg = (1.0 + 0.1 * np.random.default_rng(5).standard_normal(HD)).astype(np.float32)
    kg = (1.0 + 0.1 * np.random.default_rng(6).standard_normal(HD)).astype(np.float32)
    qgd, kgd = torch.from_numpy(qg).to(DEV), torch.from_numpy(kg).to(DEV)
    rope = m3.rope_table(max_pos)
    kc, vc = fill_cache(B, n_kv, max_pos, max_pos, 40 + B, 1.0)
    k1, v1, k2, v2 = dev(kc), dev(vc), dev(kc), dev(vc)
    for pos in (0, 5, 63, 64, 250, 399):
        qkv = dev(rnd_bf16((B, ldqkv), 600 + pos, 1.5))
        q = m3.qk_norm_rope(qkv, n_q, n_kv, qgd, kgd, rope, pos, k1, v1)
        a = m3.decode_attention(q, n_q, n_kv, k1, v1, pos + 1)
        b = m3.decode_attention_step(qkv, n_q, n_kv, qgd, kgd, rope, pos, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(a, b), pos
        assert torch.equal(k1, k2) and torch.equal(v1, v2), pos


# ---- the prompt's attention: S sequences of L positions at once ----------------
def _prompt_case(S, L, n_q, n_kv, pos_base, max_pos, seed):
    ldqkv = (n_q + 2 * n_kv) * HD
    qkv = rnd_bf16((S * L, ldqkv), seed, 1.5)
    qg = (1.0 + 0.1 * np.random.default_rng(seed + 1).standard_normal(HD)).astype(np.float32)
    kg = (1.0 + 0.1 * np.random.default_rng(seed + 2).standard_normal(HD)).astype(np.float32)
    # earlier positions (a previous chunk of the prompt) hold the same seeded values on both sides
    kc, vc = fill_cache(S, n_kv, max_pos, pos_base, seed + 3, 1.0)
    return qkv, qg, kg, kc, vc


def _oracle_prompt(qkv, S, L, n_q, n_kv, qg, kg, pos_base, kc, vc, max_pos):
    """The per-row oracle functions, row by row in position order: each row's
    norm + RoPE writes its cache slot, then it attends over the positions so far."""
    rope = O.rope_table(max_pos)
    q = np.empty((S * L, n_q * HD), np.uint16)
    out = np.empty_like(q)
    for s in range(S):
        for t in range(L):
            r = s * L + t
            q[r] = O.qk_norm_rope(qkv[r:r + 1], n_q, n_kv, qg, kg, 1e-6, rope, pos_base + t,
                                  kc[s:s + 1], vc[s:s + 1])[0]
            out[r] = O.decode_attention(q[r:r + 1], kc[s:s + 1], vc[s:s + 1], pos_base + t + 1,
                                        n_q, n_kv)[0]
    return q, out


@pytest.mark.parametrize("S,L,n_q,n_kv,pos_base", [(2, 37, 32, 8, 0), (2, 50, 32, 8, 100),
                                                    (1, 130, 16, 16, 3), (3, 7, 8, 4, 250)])
def test_prompt_attention_matches_the_rows_one_by_one(S, L, n_q, n_kv, pos_base):
    max_pos = pos_base + L + 5
    qkv, qg, kg, kc, vc = _prompt_case(S, L, n_q, n_kv, pos_base, max_pos, 40 + L)
    kd, vd = dev(kc), dev(vc)
    q = m3.prefill_qk_norm_rope(dev(qkv), S, n_q, n_kv, torch.from_numpy(qg).to(DEV),
                                torch.from_numpy(kg).to(DEV), m3.rope_table(max_pos), pos_base,
                                kd, vd)
    out = m3.prefill_attention(q, S, n_q, n_kv, kd, vd, pos_base)
    torch.cuda.synchronize()
    okc, ovc = kc.copy(), vc.copy()
    oq, oout = _oracle_prompt(qkv, S, L, n_q, n_kv, qg, kg, pos_base, okc, ovc, max_pos)
    new = slice(pos_base, pos_base + L)
    P.check_bf16_vs_bf16(synth.bits(q), oq, width=HD)
    gk, gv = synth.bits(kd), synth.bits(vd)
    P.check_bf16_vs_bf16(gk[:, :, new], okc[:, :, new], width=HD)
    assert np.array_equal(gv, ovc)
    assert np.array_equal(gk[:, :, :pos_base], kc[:, :, :pos_base])    # earlier slots untouched
    # each side attends with its own q and keys, which may differ by a bf16 ulp,
    # so the outputs get a wider row-scaled term than a single rounding
    P.check_bf16_vs_bf16(synth.bits(out), oout, agree=0.98, rel=1e-2, width=HD)


def test_prompt_then_decode_steps():
    """A 24-position prompt for 2 sequences fills the caches; three decode
    steps at positions 24, 25, 26 then attend over prompt and steps alike."""
    S, L, n_q, n_kv, max_pos = 2, 24, 32, 8, 32
    qkv, qg, kg, kc, vc = _prompt_case(S, L, n_q, n_kv, 0, max_pos, 77)
    qgd, kgd = torch.from_numpy(qg).to(DEV), torch.from_numpy(kg).to(DEV)
    rope = m3.rope_table(max_pos)
    kd, vd = dev(kc), dev(vc)
    q = m3.prefill_qk_norm_rope(dev(qkv), S, n_q, n_kv, qgd, kgd, rope, 0, kd, vd)
    m3.prefill_attention(q, S, n_q, n_kv, kd, vd, 0)
    okc, ovc = kc.copy(), vc.copy()
    _oracle_prompt(qkv, S, L, n_q, n_kv, qg, kg, 0, okc, ovc, max_pos)
    orope = O.rope_table(max_pos)
    for pos in (24, 25, 26):
        step = rnd_bf16((S, (n_q + 2 * n_kv) * HD), 900 + pos, 1.5)
        qs = m3.qk_norm_rope(dev(step), n_q, n_kv, qgd, kgd, rope, pos, kd, vd)
        o = m3.decode_attention(qs, n_q, n_kv, kd, vd, pos + 1)
        torch.cuda.synchronize()
        oq = O.qk_norm_rope(step, n_q, n_kv, qg, kg, 1e-6, orope, pos, okc, ovc)
        P.check_bf16_vs_bf16(synth.bits(o), O.decode_attention(oq, okc, ovc, pos + 1, n_q, n_kv),
                             agree=0.97, width=HD)
