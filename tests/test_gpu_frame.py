"""GPU parity of whole decode frames (DiffSynth-Studio MiniMax-Music3 stage 2:
body -> sliced lm_head draw -> depth decoder draws -> fed-back frame
embedding) against the oracle on a small model of the same structure, plus
graph replay, resume and the GPU-side frame bookkeeping (TensorFold PR #987:
position and count advance on the GPU; the host reads tokens every 16
frames)."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import configs, runtime, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"

MARGIN = 0.05     # z margin below which a draw may legitimately differ


@pytest.fixture(scope="module", params=["A", "B", "C"])
def small(request):
    cfg = configs.config("frame-small")
    p = configs.PRESETS[request.param]
    md_dev = synth.make_model(cfg, **p, seed=21, device="cpu")
    md_np = synth.model_to_numpy(md_dev)
    md_gpu = _to(md_dev, DEV)
    dm = runtime.DecodeModel(md_gpu, seed=5, temperature=1.0)
    om = O.OracleModel(md_np)
    return cfg, dm, om


def _to(v, dev):
    if isinstance(v, torch.Tensor):
        return v.to(dev)
    if isinstance(v, list):
        return [_to(x, dev) for x in v]
    if isinstance(v, dict):
        return {k: _to(x, dev) for k, x in v.items()}
    return v


def _check_frame(codes, xn, hbody, o_codes, o_xn, o_tr, body_tol=3e-2):
    sure = o_tr["zgap"] > MARGIN
    assert np.all((codes == o_codes)[sure]), (codes, o_codes)
    hb = O.bf16_to_f64(hbody)
    ref = O.bf16_to_f64(o_tr["h_body"])
    assert np.max(np.abs(hb - ref) / P.row_rms(ref)) < body_tol
    rows = np.all(codes == o_codes, 1)
    if rows.any():
        a = O.bf16_to_f64(xn[rows])
        b = O.bf16_to_f64(o_xn[rows])
        assert np.all(np.abs(a - b) <= 2 * P.half_ulp(b) + 1e-6 * P.row_rms(b))


@pytest.mark.parametrize("B", [1, 3])
def test_frames_match_oracle(small, B):
    cfg, dm, om = small
    x0 = synth.activations(B, cfg["H"], 40 + B)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=3)
    x = synth.bits(x0)
    for f in range(3, 6):
        st.decode()
        torch.cuda.synchronize()
        codes = st.codes.cpu().numpy()
        o_codes, o_xn, o_tr = O.decode_frame(om, x, seed=5, frame=f, trace=True)
        _check_frame(codes, synth.bits(st.x), synth.bits(st.h), o_codes, o_xn, o_tr)
        # continue from the oracle's own feedback (teacher forcing of the next frame input
        # only where the GPU agreed; otherwise stop comparing this row)
        if not np.array_equal(codes, o_codes):
            break
        x = o_xn
        st.x.copy_(synth.from_bits(x, DEV))
    assert int(st.frame.item()) >= 4


def test_graph_replay_equals_eager_and_resume(small):
    cfg, dm, om = small
    B = 2
    x0 = synth.activations(B, cfg["H"], 77).to(DEV)
    eager = runtime.FrameState(dm, B, x0, frame0=0)
    seq = []
    for _ in range(5):
        eager.decode()
        seq.append(eager.codes.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graphed = runtime.FrameState(dm, B, x0, frame0=0)
    with torch.cuda.stream(s):
        graphed.capture(s)
        got = []
        for _ in range(5):
            graphed.replay(s)
            s.synchronize()
            got.append(graphed.codes.clone())
            torch.cuda.synchronize()
    for a, b in zip(seq, got):
        assert torch.equal(a, b)
    assert torch.equal(eager.x, graphed.x)
    # resume: frames 0..4 straight == frames 0..2, then a fresh state from frame 3's input
    split = runtime.FrameState(dm, B, x0, frame0=0)
    for _ in range(3):
        split.decode()
    x3 = split.x.clone()
    resumed = runtime.FrameState(dm, B, x3, frame0=3)
    for k in range(3, 5):
        resumed.decode()
        torch.cuda.synchronize()
        assert torch.equal(resumed.codes, seq[k])
    # ring: frame f's codes in slot f % 16
    ring = eager.ring.cpu()
    for f in range(5):
        assert torch.equal(ring[f], seq[f].cpu())
    assert int(eager.frame.item()) == 5
    graphed.release()


def test_fused_draws_equal_standalone_sampler(small):
    """The draws finished inside the frame (sampling epilogue + gather
    prologue) equal m3_gumbel_argmax run on the same frame's logits."""
    from autoregressive_audio_lm_amd import m3
    cfg, dm, om = small
    B = 3
    x0 = synth.activations(B, cfg["H"], 99).to(DEV)
    st = runtime.FrameState(dm, B, x0, frame0=11)
    st.decode()
    torch.cuda.synchronize()
    base = cfg["vocab_base"]
    c0 = m3.gumbel_argmax(st.logits, seed=5, frame=11, draw=0, index_base=base,
                          valid=(base, base + cfg["V0"]))
    assert torch.equal(c0, st.codes[:, 0])
    dl = st.view("dlogits", torch.float32, cfg["code_vocab"])
    c7 = m3.gumbel_argmax(dl, seed=5, frame=11, draw=cfg["n_codebooks"] - 1)
    assert torch.equal(c7, st.codes[:, cfg["n_codebooks"] - 1])


def test_frame_repeat_byte_identical(small):
    cfg, dm, om = small
    B = 3
    x0 = synth.activations(B, cfg["H"], 88).to(DEV)
    a = runtime.FrameState(dm, B, x0, frame0=0)
    b = runtime.FrameState(dm, B, x0, frame0=0)
    a.decode()
    b.decode()
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes)
    assert a.state.cpu().numpy().tobytes() == b.state.cpu().numpy().tobytes()


def _same_frame(a, b):
    assert torch.equal(a.codes, b.codes)
    for name in ("x", "h", "logits"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.ring, b.ring)
    assert int(a.frame.item()) == int(b.frame.item())


@pytest.mark.parametrize("B", [1, 3, 8, 16])
def test_persistent_frame_equals_eager(small, B):
    """One cooperative launch per frame gives the eager frame's bytes (codes,
    fed-back input, residual stream, logits, ring, counter), also when eager
    and persistent frames alternate on one state."""
    cfg, dm, om = small
    x0 = synth.activations(B, cfg["H"], 300 + B).to(DEV)
    eager = runtime.FrameState(dm, B, x0, frame0=2)
    pers = runtime.FrameState(dm, B, x0, frame0=2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pers.persistent_create(s)
        for _ in range(3):
            eager.decode(s)
            pers.persistent_launch(s)
            s.synchronize()
            assert int(pers.err.item()) == 0
            _same_frame(eager, pers)
        # alternate paths on the persistent state
        pers.decode(s)
        eager.decode(s)
        pers.persistent_launch(s)
        eager.decode(s)
        s.synchronize()
        assert int(pers.err.item()) == 0
        _same_frame(eager, pers)
    pers.release()


# ------------------------------------------------ the reference's draw ----
@pytest.fixture(scope="module")
def guided():
    """The frame in the reference's draw mode (DiffSynth-Studio MiniMax-Music3
    stage 2: guidance 1.5 over each (conditional, unconditional) row pair,
    top-k 50, one draw per song taken by both rows)."""
    cfg = configs.config("frame-small")
    md_dev = synth.make_model(cfg, **configs.PRESETS["A"], seed=23, device="cpu")
    md_np = synth.model_to_numpy(md_dev)
    dm = runtime.DecodeModel(_to(md_dev, DEV), seed=5, temperature=1.0, cfg_scale=1.5, top_k=50)
    om = O.OracleModel(md_np, cfg_scale=1.5, top_k=50)
    return cfg, dm, om


def test_guided_frames_match_oracle(guided):
    cfg, dm, om = guided
    B = 4
    x0 = synth.activations(B, cfg["H"], 61)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=7)
    x = synth.bits(x0)
    for f in range(7, 10):
        st.decode()
        torch.cuda.synchronize()
        codes = st.codes.cpu().numpy()
        assert np.array_equal(codes[0::2], codes[1::2])
        o_codes, o_xn, o_tr = O.decode_frame(om, x, seed=5, frame=f, trace=True)
        _check_frame(codes, synth.bits(st.x), synth.bits(st.h), o_codes, o_xn, o_tr)
        if not np.array_equal(codes, o_codes):
            break
        x = o_xn
        st.x.copy_(synth.from_bits(x, DEV))
    assert int(st.frame.item()) >= 8


def test_guided_graph_replay_equals_eager_and_persistent_refused(guided):
    from autoregressive_audio_lm_amd import _lib
    cfg, dm, om = guided
    B = 6
    x0 = synth.activations(B, cfg["H"], 62).to(DEV)
    eager = runtime.FrameState(dm, B, x0, frame0=0)
    seq = []
    for _ in range(4):
        eager.decode()
        seq.append(eager.codes.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graphed = runtime.FrameState(dm, B, x0, frame0=0)
    with torch.cuda.stream(s):
        graphed.capture(s)
        for k in range(4):
            graphed.replay(s)
            s.synchronize()
            assert torch.equal(graphed.codes, seq[k])
            torch.cuda.synchronize()
    assert torch.equal(eager.x, graphed.x)
    graphed.release()
    with pytest.raises(_lib.M3Error):
        runtime.FrameState(dm, B, x0).persistent_create()
    with pytest.raises(_lib.M3ValueError):
        runtime.FrameState(dm, 3, x0[:3])


# ---- frames with decode attention over the state's KV caches -----------------
ATTN_MAX_POS, ATTN_POS0 = 40, 9


@pytest.fixture(scope="module", params=["A", "C"])
def attn(request):
    cfg = configs.config("frame-small")
    p = configs.PRESETS[request.param]
    md_dev = synth.make_model(cfg, **p, seed=23, device="cpu")
    md_np = synth.model_to_numpy(md_dev)
    dm = runtime.DecodeModel(_to(md_dev, DEV), seed=5, temperature=1.0, attention=1,
                             max_pos=ATTN_MAX_POS, pos0=ATTN_POS0)
    om = O.OracleModel(md_np, attention=1, max_pos=ATTN_MAX_POS, pos0=ATTN_POS0)
    return cfg, dm, om


@pytest.mark.parametrize("B", [1, 3])
def test_attention_frames_match_oracle(attn, B):
    """Frames 0 .. 5 at body positions 9 .. 14 (the prompt's positions hold
    zeros on both sides): each side keeps its own caches; the frame input
    follows the oracle's feedback while the codes agree."""
    cfg, dm, om = attn
    om.reset_attention(B)
    x0 = synth.activations(B, cfg["H"], 50 + B)
    st = runtime.FrameState(dm, B, x0.to(DEV), frame0=0)
    x = synth.bits(x0)
    agreed = 0
    for f in range(6):
        st.decode()
        torch.cuda.synchronize()
        codes = st.codes.cpu().numpy()
        o_codes, o_xn, o_tr = O.decode_frame(om, x, seed=5, frame=f, trace=True)
        # each side attends over the keys and values of its own earlier frames,
        # so the bf16 roundings in which they differ compound from frame to frame
        _check_frame(codes, synth.bits(st.x), synth.bits(st.h), o_codes, o_xn, o_tr,
                     body_tol=3e-2 if f == 0 else 6e-2)
        if not np.array_equal(codes, o_codes):
            break
        agreed += 1
        x = o_xn
        st.x.copy_(synth.from_bits(x, DEV))
    assert agreed >= 3
    assert int(st.err.item()) == 0


def test_attention_graph_replay_equals_eager_and_persistent_refused(attn):
    from autoregressive_audio_lm_amd import _lib
    cfg, dm, om = attn
    B = 2
    x0 = synth.activations(B, cfg["H"], 63).to(DEV)
    eager = runtime.FrameState(dm, B, x0, frame0=0)
    seq = []
    for _ in range(4):
        eager.decode()
        seq.append(eager.codes.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graphed = runtime.FrameState(dm, B, x0, frame0=0)
    with torch.cuda.stream(s):
        graphed.capture(s)
        for k in range(4):
            graphed.replay(s)         # each replay reads the next position from the GPU
            s.synchronize()
            assert torch.equal(graphed.codes, seq[k])
            torch.cuda.synchronize()
    assert torch.equal(eager.x, graphed.x)
    assert torch.equal(eager.state, graphed.state)     # caches included
    graphed.release()
    with pytest.raises(_lib.M3Error):
        runtime.FrameState(dm, B, x0).persistent_create()


def test_attention_frame_past_the_cache_sets_err(attn):
    """A frame whose position reaches max_pos is refused on the GPU: it keeps
    to the last slot and flags the state's err word."""
    from autoregressive_audio_lm_amd import _lib
    cfg, dm, om = attn
    B = 1
    x0 = synth.activations(B, cfg["H"], 64).to(DEV)
    st = runtime.FrameState(dm, B, x0, frame0=ATTN_MAX_POS - ATTN_POS0 - 1)
    st.decode()
    torch.cuda.synchronize()
    assert int(st.err.item()) == 0                   # position max_pos - 1: the last slot
    st.decode()
    torch.cuda.synchronize()
    assert int(st.err.item()) == _lib.M3_ERR_ATTN_FULL
