"""Pins of the oracle's frame (DiffSynth-Studio MiniMax-Music3 article, stage
2: body -> vocab-masked lm_head draw -> depth decoder draws for the 7 residual
codebooks -> frame embedding fed back) against an independent composition
written here with torch float64 library ops, plus row independence (diffusers
issue #14486, item 4) and the weight-byte formula.  CPU only, small config."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from autoregressive_audio_lm_amd import configs, synth

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def small(oracle):
    cfg = configs.config("frame-small")
    md = synth.model_to_numpy(synth.make_model(cfg, configs.BF16, configs.BF16, configs.I8G128, seed=3))
    om = oracle.OracleModel(md)
    x = synth.bits(synth.activations(3, cfg["H"], seed=5))
    return cfg, md, om, x


def _deq(oracle, W, fmt):
    """dequantised weights via the oracle's (pinned) quantisers, as float64"""
    if fmt == configs.BF16:
        return torch.from_numpy(oracle.bf16_to_f64(W))
    if fmt == configs.I8ROW:
        q, s = oracle.quant_i8row(W)
        return torch.from_numpy(q.astype(np.float64) * s.astype(np.float64)[:, None])
    q, s = oracle.quant_i8g128(W)
    return torch.from_numpy(q.astype(np.float64) * np.repeat(s.astype(np.float64), 128, 1))


def _compose(oracle, cfg, md, x_bits, seed, frame):
    """Stage 2 of the pipeline written with torch float64 ops; bf16 rounding
    points as in the method (activations after norm, every GEMV output that is
    stored, residual sums, SwiGLU output, depth inputs, feedback)."""
    r16 = lambda t: torch.from_numpy(oracle.bf16_to_f64(oracle.f64_to_bf16(t.numpy())))
    eps = cfg["eps"]

    def norm(h, g):
        return r16(F.rms_norm(h, (h.shape[1],), torch.from_numpy(g.astype(np.float64)), eps=eps))

    def layer(h, L, fmt, nh, nkv, hd):
        a = norm(h, L["attn_norm"])
        qkv = r16(a @ _deq(oracle, L["qkv"], fmt).T)
        v = qkv[:, (nh + nkv) * hd:].reshape(-1, nkv, hd)
        o = v.repeat_interleave(nh // nkv, 1).reshape(-1, nh * hd)
        h = r16(h + r16(o @ _deq(oracle, L["o"], fmt).T))
        a = norm(h, L["ffn_norm"])
        g = r16(a @ _deq(oracle, L["gate"], fmt).T)
        u = r16(a @ _deq(oracle, L["up"], fmt).T)
        m = r16(F.silu(g) * u)
        return r16(h + r16(m @ _deq(oracle, L["down"], fmt).T))

    h = torch.from_numpy(oracle.bf16_to_f64(x_bits))
    for L in md["layers"]:
        h = layer(h, L, md["fmt_body"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"])
    h_body = h
    a = norm(h, md["final_norm"])
    logits0 = (a @ _deq(oracle, md["lm_head"], md["fmt_lm"]).T).float().numpy()
    base = cfg["vocab_base"]
    c0 = oracle.gumbel_argmax(logits0, seed=seed, frame=frame, draw=0, index_base=base,
                              valid=(base, base + cfg["V0"]))
    u = r16(a @ _deq(oracle, md["p_in"], md["fmt_depth"]).T)
    codes = [c0]
    prev = np.clip(c0 - base, 0, cfg["V0"] - 1)
    for j in range(1, cfg["n_codebooks"]):
        E = md["emb1"] if j == 1 else md["emb"][j - 2]
        d = r16(u + torch.from_numpy(oracle.bf16_to_f64(E[prev])))
        for L in md["d_layers"]:
            d = layer(d, L, md["fmt_depth"], cfg["d_heads"], cfg["d_heads"], cfg["d_head_dim"])
        ad = norm(d, md["d_final_norm"])
        lj = (ad @ _deq(oracle, md["heads"][j - 1], md["fmt_depth"]).T).float().numpy()
        cj = oracle.gumbel_argmax(lj, seed=seed, frame=frame, draw=j)
        codes.append(cj)
        prev = cj
    codes = np.stack(codes, 1)
    emb = oracle.bf16_to_f64(md["tok_emb_audio"][np.clip(codes[:, 0] - base, 0, cfg["V0"] - 1)])
    for j in range(1, cfg["n_codebooks"]):
        emb = emb + oracle.bf16_to_f64(md["audio_emb"][j - 1][codes[:, j]])
    x_next = oracle.f64_to_bf16(emb / np.sqrt(cfg["n_codebooks"]))
    return codes, x_next, oracle.f64_to_bf16(h_body.numpy()), logits0


def test_frame_matches_independent_composition(oracle, small):
    cfg, md, om, x = small
    codes, xn, tr = oracle.decode_frame(om, x, seed=9, frame=4, trace=True)
    c2, xn2, hb2, lg2 = _compose(oracle, cfg, md, x, seed=9, frame=4)
    # float64 sums in a different order can flip a bf16 rounding; compare
    # with a bound of a few bf16 ulps relative to each row's rms
    hb = oracle.bf16_to_f64(tr["h_body"])
    rms = np.sqrt((hb ** 2).mean(1, keepdims=True))
    assert np.max(np.abs(hb - oracle.bf16_to_f64(hb2)) / rms) < 2e-2
    assert np.mean(tr["h_body"] == hb2) > 0.99
    rmsl = np.sqrt((lg2.astype(np.float64) ** 2).mean(1, keepdims=True))
    assert np.max(np.abs(tr["logits0"] - lg2) / rmsl) < 1e-2
    # decisions agree wherever the oracle's own margin is not razor thin
    sure = tr["zgap"] > 1e-2
    assert np.all((codes == c2)[sure])
    assert sure.mean() > 0.9
    rows = np.all(codes == c2, 1)
    assert np.array_equal(xn[rows], xn2[rows])


def test_frame_rows_independent(oracle, small):
    cfg, md, om, x = small
    codes, xn = oracle.decode_frame(om, x, seed=9, frame=4)
    # the batch row index keys the noise, so the invariant is per row: row 0
    # of a B=3 batch equals a B=1 batch, and changing the other rows leaves it
    c1, x1 = oracle.decode_frame(om, x[:1], seed=9, frame=4)
    assert np.array_equal(c1[0], codes[0]) and np.array_equal(x1[0], xn[0])
    xq = x.copy()
    xq[1:] = x[1:][:, ::-1]
    cq, xnq = oracle.decode_frame(om, xq, seed=9, frame=4)
    assert np.array_equal(cq[0], codes[0]) and np.array_equal(xnq[0], xn[0])
    assert not np.array_equal(cq[1:], codes[1:])


def test_frame_codes_in_range(oracle, small):
    cfg, md, om, x = small
    for f in range(3):
        codes, xn = oracle.decode_frame(om, x, seed=1, frame=f)
        assert np.all((codes[:, 0] >= cfg["vocab_base"]) & (codes[:, 0] < cfg["vocab_base"] + cfg["V0"]))
        assert np.all((codes[:, 1:] >= 0) & (codes[:, 1:] < cfg["code_vocab"]))
        assert np.all(np.isfinite(oracle.bf16_to_f64(xn)))


@pytest.mark.parametrize("preset", ["A", "B", "C"])
def test_weight_bytes_formula_counts_the_arrays(oracle, preset):
    """The per-frame weight-byte formula equals the byte count of the arrays
    a frame actually reads (quantised by the oracle's pinned quantisers)."""
    cfg = configs.config("frame-small")
    p = configs.PRESETS[preset]
    md = synth.model_to_numpy(synth.make_model(cfg, **p, seed=1))

    def nbytes(W, fmt):
        if fmt == configs.BF16:
            return W.nbytes
        q, s = {configs.I8ROW: oracle.quant_i8row, configs.I8G128: oracle.quant_i8g128,
                configs.FP8ROW: oracle.quant_fp8row}[fmt](W)
        return q.nbytes + s.nbytes

    def layer_bytes(L, fmt):
        return (sum(nbytes(L[k], fmt) for k in ("qkv", "o", "gate", "up", "down"))
                + L["attn_norm"].nbytes + L["ffn_norm"].nbytes)

    total = sum(layer_bytes(L, p["fmt_body"]) for L in md["layers"]) + md["final_norm"].nbytes
    total += nbytes(md["lm_head"], p["fmt_lm"]) + nbytes(md["p_in"], p["fmt_depth"])
    step = sum(layer_bytes(L, p["fmt_depth"]) for L in md["d_layers"]) + md["d_final_norm"].nbytes
    total += sum(step + nbytes(h, p["fmt_depth"]) for h in md["heads"])
    assert oracle.frame_weight_bytes(cfg, **p) == total


def test_lm_head_bytes_printed_on_the_page(oracle):
    with open(os.path.join(HERE, "golden", "frame_weight_bytes.json")) as f:
        gold = json.load(f)
    cfg = configs.config("frame-full")
    # the full bf16 lm_head the reference pipeline reads per frame: rows up to
    # the end of the audio range, hidden 4096, 2 bytes -> the printed 1.38 GB
    rows = cfg["vocab_base"] + cfg["V0"]
    assert round(rows * cfg["H"] * 2 / 1e9, 2) == gold["lm_head_full_gb_printed"]
