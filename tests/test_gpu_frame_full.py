"""Whole decode frames at the full model size (36-layer Qwen3-8B-shaped body,
16384-row lm_head slice, 4-layer depth decoder x 7 codebooks), run the way
bench.py times them (one captured HIP graph replayed per frame), against the
oracle's frame on the same bf16 weights (DiffSynth-Studio MiniMax-Music3,
stage 2).

A 36-layer bf16 stack turns every differing bf16 rounding into ulp-sized
differences that accumulate along the residual stream: two correct
implementations agree only up to that envelope, not bit for bit.  The
envelope is measured on the oracle itself: the same frame from inputs that
differ in the last bit of one element.  The GPU frame must stay within a
small multiple of it (a wrong index or a dropped term is orders of magnitude
outside), and every draw that is stable under those perturbations, with a
margin, must be identical.  Tight per-operation parity at these shapes is the
job of the GEMV tests; this one checks the frame as a whole."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import configs, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
ENVELOPE_FACTOR = 4.0
FLIPS = ((0, 17), (0, 2049))       # (row, column) whose lowest mantissa bit is flipped


def _dev(a_bits, ref_bits):
    a, r = O.bf16_to_f64(a_bits), O.bf16_to_f64(ref_bits)
    return float(np.max(np.abs(a - r) / P.row_rms(r)))


@pytest.mark.parametrize("preset,B", [("A", 1), ("B", 2)])
def test_full_size_frame_within_rounding_envelope(preset, B):
    cfg = configs.config("frame-full")
    p = configs.PRESETS[preset]
    md = synth.make_model(cfg, **p, seed=13, device=DEV)
    md_np = synth.model_to_numpy(md)
    dm = runtime.DecodeModel(md, seed=9, free_sources=True)
    del md
    torch.cuda.empty_cache()
    om = O.OracleModel(md_np)
    del md_np
    f = 7
    x0 = synth.activations(B, cfg["H"], 500)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=f)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.capture(s)
        st.replay(s)
        s.synchronize()
    torch.cuda.synchronize()
    codes = st.codes.cpu().numpy()
    h_gpu = synth.bits(st.h)
    lg_gpu = st.logits.cpu().numpy().astype(np.float64)
    frame_after = int(st.frame.item())
    st.release()

    x = synth.bits(x0)
    o_codes, o_xn, tr = O.decode_frame(om, x, seed=9, frame=f, trace=True)
    env_h, env_l, stable = 0.0, 0.0, np.ones_like(o_codes, dtype=bool)
    for (b, k) in FLIPS:
        xp = x.copy()
        xp[b % B, k] ^= 1
        c2, _, t2 = O.decode_frame(om, xp, seed=9, frame=f, trace=True)
        env_h = max(env_h, _dev(t2["h_body"], tr["h_body"]))
        env_l = max(env_l, float(np.max(np.abs(t2["logits0"].astype(np.float64) - tr["logits0"]))))
        stable &= c2 == o_codes
    dev_h = _dev(h_gpu, tr["h_body"])
    dev_l = float(np.max(np.abs(lg_gpu - tr["logits0"])))
    print(f"preset {preset} B={B}: h_body dev {dev_h:.3e} (envelope {env_h:.3e}); "
          f"logits dev {dev_l:.3e} (envelope {env_l:.3e}); codes {codes.tolist()} "
          f"oracle {o_codes.tolist()}", flush=True)

    assert frame_after == f + 1
    assert np.all((codes[:, 0] >= cfg["vocab_base"]) & (codes[:, 0] < cfg["vocab_base"] + cfg["V0"]))
    assert np.all((codes[:, 1:] >= 0) & (codes[:, 1:] < cfg["code_vocab"]))
    assert dev_h <= ENVELOPE_FACTOR * env_h
    assert dev_l <= ENVELOPE_FACTOR * env_l
    # a draw is compared where the oracle's own perturbed frames agree and its
    # winning margin exceeds the logit envelope
    sure = stable & (tr["zgap"] > ENVELOPE_FACTOR * env_l)
    sure[:, 1:] &= sure[:, :1]           # the depth chain is conditioned on the semantic code
    assert np.all((codes == o_codes)[sure])


@pytest.mark.parametrize("preset,B", [("A", 1), ("A", 6), ("B", 2), ("C", 1)])
def test_full_size_persistent_equals_graph(preset, B):
    """The persistent frame (one cooperative launch, tagged intermediate
    streams) and the graph-replayed frame give identical bytes at the full
    model size, up to B = 6, the largest row count whose down-projection
    operand (K = 12288) is staged in LDS."""
    cfg = configs.config("frame-full")
    md = synth.make_model(cfg, **configs.PRESETS[preset], seed=17, device=DEV)
    dm = runtime.DecodeModel(md, seed=4, free_sources=True)
    del md
    torch.cuda.empty_cache()
    x0 = synth.activations(B, cfg["H"], 900, device=DEV)
    g = runtime.FrameState(dm, B, x0, frame0=40)
    p = runtime.FrameState(dm, B, x0, frame0=40)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture(s)
        p.persistent_create(s)
        for _ in range(2):
            g.replay(s)
            p.persistent_launch(s)
            s.synchronize()
            assert int(p.err.item()) == 0
            assert torch.equal(g.codes, p.codes)
            for name in ("x", "h", "logits"):
                assert torch.equal(getattr(g, name), getattr(p, name)), name
            assert torch.equal(g.ring, p.ring)
    g.release()
    p.release()


@pytest.mark.parametrize("preset,B,frames", [("A", 1, 300), ("B", 2, 150)])
def test_full_size_persistent_equals_graph_over_many_frames(preset, B, frames):
    """A chained run: every frame feeds the next (codes -> embeddings -> x),
    the persistent frame and the graph-replayed frame stay byte-identical
    frame after frame, and the persistent launches never give up waiting.
    300 launches take the 16-bit tags of the tagged streams (launch counter
    * 512 + phase + 1) through their wrap-around twice."""
    cfg = configs.config("frame-full")
    md = synth.make_model(cfg, **configs.PRESETS[preset], seed=23, device=DEV)
    dm = runtime.DecodeModel(md, seed=6, free_sources=True)
    del md
    torch.cuda.empty_cache()
    x0 = synth.activations(B, cfg["H"], 902, device=DEV)
    g = runtime.FrameState(dm, B, x0, frame0=3)
    p = runtime.FrameState(dm, B, x0, frame0=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture(s)
        p.persistent_create(s)
        for f in range(frames):
            g.replay(s)
            p.persistent_launch(s)
            s.synchronize()
            assert int(p.err.item()) == 0, f
            assert torch.equal(g.codes, p.codes), f
            if f % 50 == 49 or f == frames - 1:
                for name in ("x", "h", "logits"):
                    assert torch.equal(getattr(g, name), getattr(p, name)), (f, name)
                assert torch.equal(g.ring, p.ring), f
                assert int(g.frame.item()) == int(p.frame.item()) == 3 + f + 1
    g.release()
    p.release()


def test_full_size_persistent_refuses_unstaged_operands():
    """At B = 16 the body down projection's operand does not fit LDS: the
    persistent frame is refused (the graph-replayed frame serves it)."""
    from autoregressive_audio_lm_amd import _lib
    cfg = configs.config("frame-full", n_layers=1)
    md = synth.make_model(cfg, **configs.PRESETS["A"], seed=17, device=DEV)
    dm = runtime.DecodeModel(md, seed=4, free_sources=True)
    st = runtime.FrameState(dm, 16, synth.activations(16, cfg["H"], 901, device=DEV))
    with pytest.raises(_lib.M3ValueError):
        st.persistent_create()


def test_full_size_attention_frame_within_rounding_envelope():
    """The frame with decode attention at the full model size and position
    1797 (the end of a 60 s song): both sides start from the same seeded
    keys and values at the 1797 earlier positions of every layer's cache; the
    GPU's graph-replayed frame stays within the oracle's rounding envelope
    and its stable draws are identical."""
    cfg = configs.config("frame-full")
    B, max_pos, pos0 = 1, 2048, 1797
    md = synth.make_model(cfg, **configs.PRESETS["A"], seed=19, device=DEV)
    md_np = synth.model_to_numpy(md)
    dm = runtime.DecodeModel(md, seed=9, free_sources=True, attention=1, max_pos=max_pos,
                             pos0=pos0)
    del md
    torch.cuda.empty_cache()
    om = O.OracleModel(md_np, attention=1, max_pos=max_pos, pos0=pos0)
    del md_np
    om.reset_attention(B)
    x0 = synth.activations(B, cfg["H"], 510)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=0)
    L, nkv = cfg["n_layers"], cfg["n_kv_heads"]
    n = L * B * nkv * max_pos * 128
    for name, seed in (("kcache", 700), ("vcache", 701)):
        off = getattr(st.layout, name)
        cache = st.state[off:off + 2 * n].view(torch.bfloat16).view(L, B, nkv, max_pos, 128)
        cache[:, :, :, :pos0] = synth.normal_bf16((L, B, nkv, pos0, 128), seed, 1.0, DEV)
        host = synth.bits(cache)
        for l in range(L):
            getattr(om, name)[l][...] = host[l]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.capture(s)
        st.replay(s)
        s.synchronize()
    torch.cuda.synchronize()
    codes = st.codes.cpu().numpy()
    h_gpu = synth.bits(st.h)
    lg_gpu = st.logits.cpu().numpy().astype(np.float64)
    assert int(st.err.item()) == 0
    st.release()

    x = synth.bits(x0)
    o_codes, _, tr = O.decode_frame(om, x, seed=9, frame=0, trace=True)
    env_h, env_l, stable = 0.0, 0.0, np.ones_like(o_codes, dtype=bool)
    for (b, k) in FLIPS:
        xp = x.copy()
        xp[b % B, k] ^= 1
        c2, _, t2 = O.decode_frame(om, xp, seed=9, frame=0, trace=True)
        env_h = max(env_h, _dev(t2["h_body"], tr["h_body"]))
        env_l = max(env_l, float(np.max(np.abs(t2["logits0"].astype(np.float64) - tr["logits0"]))))
        stable &= c2 == o_codes
    dev_h = _dev(h_gpu, tr["h_body"])
    dev_l = float(np.max(np.abs(lg_gpu - tr["logits0"])))
    print(f"attention frame at position {pos0}: h_body dev {dev_h:.3e} (envelope {env_h:.3e}); "
          f"logits dev {dev_l:.3e} (envelope {env_l:.3e}); codes {codes.tolist()} "
          f"oracle {o_codes.tolist()}", flush=True)
    assert dev_h <= ENVELOPE_FACTOR * env_h
    assert dev_l <= ENVELOPE_FACTOR * env_l
    sure = stable & (tr["zgap"] > ENVELOPE_FACTOR * env_l)
    sure[:, 1:] &= sure[:, :1]
    assert np.all((codes == o_codes)[sure])
