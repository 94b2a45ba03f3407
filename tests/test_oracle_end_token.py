"""Pins of the oracle frame's end token (DiffSynth-Studio MiniMax-Music3
article, stage 2: the semantic draw is masked to the audio codes and the end
token 151670, and a song ends when it is drawn).  The sliced draw over the
codes plus the end token's own lm_head row is pinned against the same draw
over the whole 200000-id vocabulary with every other id masked (the noise is
keyed by absolute id); an end token whose logit can never win leaves the
frame exactly as without it; one that always wins is drawn by every row, and
the frame then embeds code 0's rows (its defined lockstep continuation).
CPU only."""
import numpy as np
import pytest

from autoregressive_audio_lm_amd import configs, synth


def _a_rows(O, om, md, x):
    """The normalised body output of a frame from x (the lm_head's operand)."""
    _, _, tr = O.decode_frame(om, x, seed=3, frame=0, trace=True)
    return O.bf16_to_f64(O.rmsnorm(tr["h_body"], md["final_norm"], md["cfg"]["eps"]))


@pytest.fixture(scope="module")
def small(oracle):
    cfg = configs.config("frame-small")
    md = synth.model_to_numpy(synth.make_model(cfg, **configs.PRESETS["A"], seed=41))
    x = synth.bits(synth.activations(4, cfg["H"], 77))
    return cfg, md, x


def _with_end_row(md, row):
    md2 = dict(md)
    md2["lm_end"] = row.reshape(1, -1)
    return md2


def test_end_token_draw_equals_the_masked_full_vocabulary_draw(oracle, small):
    O = oracle
    cfg, md, x = small
    a = _a_rows(O, O.OracleModel(md), md, x)
    # an end row that wins for rows 0 and 2 and competes nowhere else
    md2 = _with_end_row(md, O.f64_to_bf16(0.1 * (a[0] + a[2] - a[1] - a[3])))
    om = O.OracleModel(md2, end_token=True)
    codes, _, tr = O.decode_frame(om, x, seed=3, frame=0, trace=True)
    lg = tr["logits0"]
    assert lg.shape == (4, cfg["V0"] + 1)
    V, base, end = cfg["vocab"], cfg["vocab_base"], cfg["end_token"]
    full = np.full((4, V), -np.inf, np.float32)
    full[:, end] = lg[:, 0]
    full[:, base:base + cfg["V0"]] = lg[:, 1:]
    want = O.gumbel_argmax(full, seed=3, frame=0, draw=0, index_base=0)
    assert np.array_equal(codes[:, 0], want)
    assert codes[0, 0] == end and codes[2, 0] == end
    assert codes[1, 0] != end and codes[3, 0] != end


@pytest.mark.parametrize("xseed", [77, 78])
def test_unreachable_end_token_changes_nothing(oracle, small, xseed):
    O = oracle
    cfg, md, _ = small
    x = synth.bits(synth.activations(4, cfg["H"], xseed))
    om0 = O.OracleModel(md)
    a = _a_rows(O, om0, md, x)
    # a logit of about -0.5 |a_b|^2 for every row: far below every code's
    md2 = _with_end_row(md, O.f64_to_bf16(-0.5 * a.sum(0)))
    om1 = O.OracleModel(md2, end_token=True)
    c0, x0 = O.decode_frame(om0, x, seed=3, frame=0)
    c1, x1 = O.decode_frame(om1, x, seed=3, frame=0)
    assert np.array_equal(c0, c1) and np.array_equal(x0, x1)


def test_end_token_drawn_everywhere_embeds_code_zero(oracle, small):
    O = oracle
    cfg, md, x = small
    a = _a_rows(O, O.OracleModel(md), md, x)
    md2 = _with_end_row(md, O.f64_to_bf16(0.5 * a.sum(0)))
    om = O.OracleModel(md2, end_token=True)
    codes, xn = O.decode_frame(om, x, seed=3, frame=0)
    assert np.all(codes[:, 0] == cfg["end_token"])
    # the depth step 1 input and the frame embedding take code 0's rows
    zero = codes.copy()
    zero[:, 0] = cfg["vocab_base"]
    assert np.array_equal(O.feedback(om, codes), O.feedback(om, zero))
    assert np.array_equal(xn, O.feedback(om, codes))
    u = np.zeros((4, cfg["D"]), np.uint16)
    assert np.array_equal(O.step_input(om, 1, codes, u), O.step_input(om, 1, zero, u))


def test_frames_generated_from_stop_words():
    """The host's reading of the stop words: frames before the end token, -1
    while running, and an end token at the first frame is an error."""
    from autoregressive_audio_lm_amd import runtime
    n = runtime.frames_generated([0, 8, 13, 0], frame0=5)
    assert n.tolist() == [-1, 2, 7, -1]
    with pytest.raises(runtime.NoFramesError):
        runtime.frames_generated([0, 6], frame0=5)
