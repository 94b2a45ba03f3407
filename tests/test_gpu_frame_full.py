"""Whole decode frames at the full model size (36-layer Qwen3-8B-shaped body,
16384-row lm_head slice, 4-layer depth decoder x 7 codebooks), run the way
bench.py times them (a replayed HIP graph, or one persistent launch), against
the oracle (DiffSynth-Studio MiniMax-Music3, stage 2).

Every stage of the frame is compared with the oracle on the GPU's own input
of that stage (tests/stages.py; TensorFold PR #987, summary: parity at every
stage, teacher-forced): each body layer, the lm_head logits, the semantic
draw, the depth input projection, each depth step's input, layers, head
logits and draw, and the fed-back input.  A 36-layer bf16 stack amplifies
every differing rounding along the residual stream, so two correct
implementations run freely from the same input agree only loosely after 36
layers; stage by stage, each output is held to its own per-operation
tolerance and every draw to bit-exactness."""
import numpy as np
import pytest
import torch

import oracle as O
import stages
from autoregressive_audio_lm_amd import _lib, configs, m3, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (B, path) per preset; the persistent frame takes B <= 6 at the full shapes
CASES = {"A": [(1, "graph"), (1, "persistent"), (6, "graph"), (6, "persistent"), (16, "graph")],
         "B": [(1, "persistent"), (6, "graph"), (6, "persistent"), (16, "graph")],
         "C": [(1, "persistent"), (16, "graph")]}
# batch rows whose layer and GEMV outputs the oracle recomputes (every draw,
# step input and feedback is checked on all rows)
ROWS = {1: [0], 6: [0, 2, 5], 16: [0, 5, 10, 15]}


@pytest.fixture(scope="module", params=["A", "B", "C"])
def full(request):
    preset = request.param
    cfg = configs.config("frame-full")
    md = synth.make_model(cfg, **configs.PRESETS[preset], seed=13, device=DEV)
    md_np = synth.model_to_numpy(md)
    dm = runtime.DecodeModel(md, seed=9, free_sources=True)
    del md
    torch.cuda.empty_cache()
    om = O.OracleModel(md_np)
    yield preset, cfg, dm, om
    del dm, om
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,path", [(1, "graph"), (1, "persistent"), (6, "graph"),
                                    (6, "persistent"), (16, "graph")])
def test_full_size_frame_stages(full, B, path):
    """A full-size frame, every operation against the oracle on the GPU's own
    input of that operation (all 36 body layers, all 7 depth steps of 4
    layers, every head and draw, the feedback)."""
    preset, cfg, dm, om = full
    if (B, path) not in CASES[preset]:
        pytest.skip(f"preset {preset} runs {CASES[preset]}")
    x0 = synth.activations(B, cfg["H"], 500 + B)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=7)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        if path == "graph":
            st.capture(s)
        else:
            st.persistent_create(s)
    with torch.cuda.stream(s):
        st.replay(s) if path == "graph" else st.persistent_launch(s)
    s.synchronize()
    assert int(st.err.item()) == 0
    assert int(st.frame.item()) == 8
    got = stages.read_frame(st, tagged=path == "persistent")
    st.release()
    stats = stages.check_frame(om, got, synth.bits(x0), seed=9, frame=7, rows=ROWS[B])
    print(f"preset {preset} {path} B={B}: {stats.summary()}; codes {got['codes'][:2].tolist()}",
          flush=True)


@pytest.mark.parametrize("B", [7, 16])
def test_full_size_split_equals_one_launch(full, B):
    """From B = 7 on, the down projection's operand (K = 12288) does not fit
    LDS, and the graph frame runs it split along K (the depth decoder's down
    too from B = 14): each workgroup stages a quarter of the operand for four
    row blocks, and the last workgroup of each group of row blocks sums the
    wave partials in the one-launch kernel's order.  Every layer's output
    equals, byte for byte, the standalone GEMV call (one launch, operand read
    from memory) on the frame's own operand and residual, over two replays
    (the group counters are left at zero for the next launch); O, which is
    not split, is checked the same way."""
    preset, cfg, dm, om = full
    c = dm.config
    x0 = synth.activations(B, cfg["H"], 700 + B)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        st.capture(s)
        st.replay(s)
        st.replay(s)
    s.synchronize()
    assert int(st.frame.item()) == 5
    mlp, ho, h = st.slots("mlp"), st.slots("ho"), st.slots("h")
    with torch.cuda.stream(s):
        for l in range(c.n_layers):
            y = m3.gemv(dm.fmt_body, dm.packed_layers[l]["down"], c.hidden, c.ffn, mlp[l],
                        epi=m3.EPI_RESIDUAL, residual=ho[l], stream=s)
            s.synchronize()
            assert torch.equal(y.view(torch.int16), h[l].view(torch.int16)), l
        # O (the attention stub's V heads, 4 query heads per KV head), from
        # layer 1 on (layer 0's residual, the frame input, is overwritten by
        # the next input at the frame's end)
        qkv = st.slots("qkv")
        nq, nkv = c.n_heads * c.head_dim, c.n_kv_heads * c.head_dim
        for l in range(1, c.n_layers):
            y = m3.gemv(dm.fmt_body, dm.packed_layers[l]["o"], c.hidden, nq, qkv[l],
                        stub_group=c.n_heads // c.n_kv_heads, stub_voff=nq + nkv,
                        epi=m3.EPI_RESIDUAL, residual=h[l - 1], stream=s)
            s.synchronize()
            assert torch.equal(y.view(torch.int16), ho[l].view(torch.int16)), ("o", l)
        dmlp, hdo, hd, dqkv = st.slots("dmlp"), st.slots("hdo"), st.slots("hd"), st.slots("dqkv")
        dq = c.d_heads * c.d_head_dim
        for j in range(c.n_codebooks - 1):
            for l in range(c.d_layers):
                y = m3.gemv(dm.fmt_depth, dm.packed_dlayers[l]["down"], c.d_hidden, c.d_ffn,
                            dmlp[j, l], epi=m3.EPI_RESIDUAL, residual=hdo[j, l], stream=s)
                y2 = m3.gemv(dm.fmt_depth, dm.packed_dlayers[l]["o"], c.d_hidden, dq, dqkv[j, l],
                             stub_group=1, stub_voff=2 * dq, epi=m3.EPI_RESIDUAL,
                             residual=hd[j, l], stream=s)
                s.synchronize()
                assert torch.equal(y.view(torch.int16), hd[j, l + 1].view(torch.int16)), (j, l)
                assert torch.equal(y2.view(torch.int16), hdo[j, l].view(torch.int16)), ("do", j, l)
    st.release()
    print(f"preset {preset} B={B}: O and the split down projections equal the one-launch GEMV", flush=True)


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


def _seed_full_caches(st, cfg, B, max_pos, pos0):
    """Seeded keys and values at the positions before pos0 of every layer."""
    L, nkv = cfg["n_layers"], cfg["n_kv_heads"]
    n = L * B * nkv * max_pos * 128
    for name, seed in (("kcache", 700), ("vcache", 701)):
        off = getattr(st.layout, name)
        cache = st.state[off:off + 2 * n].view(torch.bfloat16).view(L, B, nkv, max_pos, 128)
        cache[:, :, :, :pos0] = synth.normal_bf16((L, B, nkv, pos0, 128), seed, 1.0, DEV)
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def full_attn():
    cfg = configs.config("frame-full")
    max_pos, pos0 = 2048, 1797
    md = synth.make_model(cfg, **configs.PRESETS["A"], seed=19, device=DEV)
    md_np = synth.model_to_numpy(md)
    dm = runtime.DecodeModel(md, seed=9, free_sources=True, attention=1, max_pos=max_pos,
                             pos0=pos0)
    del md
    torch.cuda.empty_cache()
    om = O.OracleModel(md_np, attention=1, max_pos=max_pos, pos0=pos0)
    yield cfg, dm, om, max_pos, pos0
    del dm, om
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["graph", "persistent"])
def test_full_size_attention_frame_stages(full_attn, path):
    """Frames with decode attention at the full model size near the end of a
    60 s song (positions 1797 and 1798): every layer's cache holds seeded keys
    and values at the earlier positions; every stage of two chained
    graph-replayed or persistent frames is compared with the oracle on the
    GPU's own input of that stage, body layers attending over the cache as it
    was before the frame plus the slot each side writes (the GPU's written
    slots compared too), depth steps over the GPU's earlier codebook
    positions."""
    cfg, dm, om, max_pos, pos0 = full_attn
    B = 1
    x0 = synth.activations(B, cfg["H"], 510)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=0)
    _seed_full_caches(st, cfg, B, max_pos, pos0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        if path == "graph":
            st.capture(s)
        else:
            st.persistent_create(s)
    x = synth.bits(x0)
    for f in (0, 1):
        before = stages.read_caches(st)
        with torch.cuda.stream(s):
            if path == "graph":
                st.replay(s)
            else:
                st.persistent_launch(s)
        s.synchronize()
        assert int(st.err.item()) == 0
        got = stages.read_frame(st, tagged=path == "persistent")
        after = stages.read_caches(st)
        stats = stages.check_frame(om, got, x, seed=9, frame=f,
                                   attn=dict(pos=pos0 + f, before=before, after=after))
        print(f"attention {path} frame at position {pos0 + f}: {stats.summary()}; codes "
              f"{got['codes'].tolist()}", flush=True)
        x = got["x"]
    st.release()


@pytest.mark.parametrize("B", [1, 2, 6])
def test_full_size_attention_persistent_equals_graph(full_attn, B):
    """Persistent and graph-replayed attention frames at the full model size
    give identical bytes (codes, the fed-back input, the body output, the
    logits and every KV cache) over three chained frames."""
    cfg, dm, om, max_pos, pos0 = full_attn
    x0 = synth.activations(B, cfg["H"], 905, device=DEV)
    g = runtime.FrameState(dm, B, x0, frame0=0)
    p = runtime.FrameState(dm, B, x0, frame0=0)
    for st in (g, p):
        _seed_full_caches(st, cfg, B, max_pos, pos0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture(s)
        p.persistent_create(s)
        for f in range(3):
            g.replay(s)
            p.persistent_launch(s)
            s.synchronize()
            assert int(p.err.item()) == 0 and int(g.err.item()) == 0
            assert torch.equal(g.codes, p.codes), f
            for name in ("x", "h", "logits"):
                assert torch.equal(getattr(g, name), getattr(p, name)), (f, name)
    lo, hi = g.layout.kcache, g.layout.attn_ws     # kcache, vcache, dkcache, dvcache
    assert torch.equal(g.state[lo:hi], p.state[lo:hi])      # every cache, every position
    g.release()
    p.release()


@pytest.mark.parametrize("B", [2, 6])
def test_full_size_song_frame_persistent_equals_graph(full_attn, B):
    """The frame a song runs at the full model size: the reference's draw
    (guidance 1.5 over each row pair, top-k 50) with decode attention near
    the end of a 60 s song; persistent frames (attention and draw phases)
    byte-identical to graph frames over three chained frames, caches
    included, and both rows of each song carry its draws."""
    cfg, dm, om, max_pos, pos0 = full_attn
    dm.set_draw(1.5, 50)
    try:
        x0 = synth.activations(B, cfg["H"], 907, device=DEV)
        g = runtime.FrameState(dm, B, x0, frame0=0)
        p = runtime.FrameState(dm, B, x0, frame0=0)
        for st in (g, p):
            _seed_full_caches(st, cfg, B, max_pos, pos0)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g.capture(s)
            p.persistent_create(s)
            for f in range(3):
                g.replay(s)
                p.persistent_launch(s)
                s.synchronize()
                assert int(p.err.item()) == 0 and int(g.err.item()) == 0
                assert torch.equal(g.codes, p.codes), f
                assert torch.equal(p.codes[0::2], p.codes[1::2]), f
                for name in ("x", "h", "logits", "dlogits"):
                    assert torch.equal(getattr(g, name), getattr(p, name)), (f, name)
        lo, hi = g.layout.kcache, g.layout.attn_ws
        assert torch.equal(g.state[lo:hi], p.state[lo:hi])
        g.release()
        p.release()
    finally:
        dm.set_draw(1.5, 0)

