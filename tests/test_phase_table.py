"""The persistent frame's phase table against the ordering its tag protocol
rests on, on the host (m3_frame_phase_table builds the table without a GPU).

Inside one persistent launch a step waits for the tags its producer writes
into the words it reads (see gemv_impl.h).  That is sound if (1) every tagged
input is written, whole, by the producer the step waits for, and that
producer comes earlier; (2) no byte is written by two steps of one frame, so
no newer tag can replace the awaited one while a reader still waits for it;
(3) what a GEMV reads untagged is written before the launch (only the frame
end, which runs after every workgroup finished every GEMV, writes it again);
(4) a frame has fewer steps than the tag period (512); (5) what an attention
step reads untagged (its KV cache) is written before the launch, by the step
itself, or by an attention step it depends on through the tags it waits for
(the depth decoder's cache, filled one position per codebook step; the kernel
gives those rows' items to the workgroup that wrote them); (6) what a guided
draw reads untagged (the logits) is written by the step right before it, for
whose every workgroup it waits."""
import ctypes

import pytest

from autoregressive_audio_lm_amd import _lib, configs, runtime

pytestmark = pytest.mark.filterwarnings("ignore")

STATE = 0x2000_0000_0000      # fake, 256-aligned device addresses: nothing is dereferenced
CODES = 0x3000_0000_0000


def fake_model(cfg: dict, preset: str):
    """An m3_model whose weight pointers are distinct fake addresses."""
    c = runtime.make_config(cfg, **configs.PRESETS[preset])
    nxt = [0x1000_0000_0000]

    def addr():
        nxt[0] += 1 << 24
        return ctypes.c_void_p(nxt[0])

    def layer():
        return _lib.LayerWeights(addr(), addr(), addr(), addr(), addr(), addr(), addr(), addr())

    keep = []
    layers = (_lib.LayerWeights * cfg["n_layers"])(*[layer() for _ in range(cfg["n_layers"])])
    dl = (_lib.LayerWeights * cfg["d_layers"])(*[layer() for _ in range(cfg["d_layers"])])
    S = cfg["n_codebooks"] - 1
    heads = (ctypes.c_void_p * S)(*[addr().value for _ in range(S)])
    emb = (ctypes.c_void_p * max(S - 1, 1))(*[addr().value for _ in range(max(S - 1, 1))])
    aemb = (ctypes.c_void_p * S)(*[addr().value for _ in range(S)])
    keep += [layers, dl, heads, emb, aemb]
    m = _lib.Model(cfg=c, layers=ctypes.cast(layers, ctypes.c_void_p), final_norm=addr(),
                   lm_head=addr(), p_in=addr(), emb1=addr(), emb=ctypes.cast(emb, ctypes.c_void_p),
                   d_layers_w=ctypes.cast(dl, ctypes.c_void_p), d_final_norm=addr(),
                   heads=ctypes.cast(heads, ctypes.c_void_p), tok_emb_audio=addr(),
                   audio_emb=ctypes.cast(aemb, ctypes.c_void_p))
    return m, keep


def phase_table(m, B):
    L = _lib.lib()
    n = L.m3_frame_phase_table(ctypes.byref(m), ctypes.c_void_p(STATE), B, ctypes.c_void_p(CODES),
                               None, 0)
    assert n > 0, n
    recs = (_lib.PhaseRecord * n)()
    assert L.m3_frame_phase_table(ctypes.byref(m), ctypes.c_void_p(STATE), B,
                                  ctypes.c_void_p(CODES), recs, n) == n
    out = []
    for r in recs:
        def regs(arr, k):
            return [dict(rows=[(g.base + i * g.stride + g.c0, g.base + i * g.stride + g.c1)
                               for i in range(g.rows)],
                         producer=g.producer, tagged=bool(g.tagged)) for g in arr[:k]]
        out.append(dict(kind=r.kind, inp=regs(r.inp, r.n_in), out=regs(r.out, r.n_out)))
    return out


def violations(recs):
    """Every breach of the ordering rules in the module docstring."""
    bad = []
    n = len(recs)
    if n >= 512:
        bad.append(f"{n} steps: tags repeat within a frame")
    if recs[-1]["kind"] != _lib.PHASE_FRAME_END or any(
            r["kind"] not in (_lib.PHASE_GEMV, _lib.PHASE_ATTENTION, _lib.PHASE_DRAW)
            for r in recs[:-1]):
        bad.append("the frame end is not the last step, or not the only one")
    # the steps each step depends on through the tags it waits for; a draw
    # (and the frame end) waits for every workgroup to finish the step before
    # it, and so for every earlier step
    anc = []
    for i, r in enumerate(recs):
        a = set(range(i)) if r["kind"] in (_lib.PHASE_DRAW, _lib.PHASE_FRAME_END) else set()
        for g in r["inp"]:
            p = g["producer"]
            if g["tagged"] and 0 <= p < i:
                a |= {p} | anc[p]
        anc.append(a)
    writes = []                              # (lo, hi, step, tagged)
    for i, r in enumerate(recs):
        for o in r["out"]:
            writes += [(lo, hi, i, o["tagged"]) for lo, hi in o["rows"]]
    ws = sorted(writes)
    for a, b in zip(ws, ws[1:]):
        if b[0] < a[1]:
            bad.append(f"bytes [{b[0]:#x}, {min(a[1], b[1]):#x}) written by steps {a[2]} and {b[2]}")
    for i, r in enumerate(recs):
        for g in r["inp"]:
            for lo, hi in g["rows"]:
                cover = [w for w in ws if w[0] < hi and lo < w[1]]
                if g["tagged"]:
                    p = g["producer"]
                    if not 0 <= p < i:
                        bad.append(f"step {i} waits for step {p}")
                    if any(w[2] != p or not w[3] for w in cover):
                        bad.append(f"step {i} reads [{lo:#x}, {hi:#x}) tagged by {p}, written by "
                                   f"{sorted({(w[2], w[3]) for w in cover})}")
                    # covered whole by the producer's tagged writes
                    pos = lo
                    for w in sorted(cover):
                        if w[0] > pos:
                            break
                        pos = max(pos, w[1])
                    if pos < hi:
                        bad.append(f"step {i} reads [{lo:#x}, {hi:#x}) that step {p} does not "
                                   f"write whole")
                elif r["kind"] == _lib.PHASE_GEMV:
                    if any(w[2] != n - 1 for w in cover):
                        bad.append(f"step {i} reads untagged bytes that step(s) "
                                   f"{sorted({w[2] for w in cover})} write in the frame")
                elif r["kind"] == _lib.PHASE_DRAW:
                    if any(w[2] != i - 1 for w in cover) or g["producer"] != i - 1:
                        bad.append(f"draw step {i} reads untagged bytes that step(s) "
                                   f"{sorted({w[2] for w in cover})} write in the frame")
                elif r["kind"] == _lib.PHASE_ATTENTION:
                    if any(w[2] != i and not (w[2] in anc[i] and
                                              recs[w[2]]["kind"] == _lib.PHASE_ATTENTION)
                           for w in cover):
                        bad.append(f"attention step {i} reads untagged bytes that step(s) "
                                   f"{sorted({w[2] for w in cover})} write in the frame")
                elif any(w[2] >= i for w in cover):
                    bad.append(f"the frame end reads bytes it writes itself")
    return bad


CASES = [("frame-small", "A", 1), ("frame-small", "A", 3), ("frame-small", "B", 6),
         ("frame-small", "C", 2), ("frame-full", "A", 1), ("frame-full", "A", 6),
         ("frame-full", "B", 2), ("frame-full", "C", 4)]


@pytest.mark.parametrize("name,preset,B", CASES)
def test_phase_table_ordering(name, preset, B):
    cfg = configs.config(name)
    m, keep = fake_model(cfg, preset)
    recs = phase_table(m, B)
    # body: 4 GEMVs per layer, the lm_head, the depth input projection, 7 steps
    # of 4 GEMVs per depth layer and a head, the frame end
    S = cfg["n_codebooks"] - 1
    assert len(recs) == 4 * cfg["n_layers"] + 2 + S * (4 * cfg["d_layers"] + 1) + 1
    assert violations(recs) == []


ATTN_CASES = [("frame-small", "A", 1, 40), ("frame-small", "A", 3, 300),
              ("frame-small", "C", 2, 64), ("frame-full", "A", 1, 2048),
              ("frame-full", "B", 6, 2048), ("frame-full", "A", 2, 100)]


@pytest.mark.parametrize("name,preset,B,max_pos", ATTN_CASES)
def test_phase_table_ordering_with_attention(name, preset, B, max_pos):
    """Frames with decode attention: an attention step per body layer and per
    depth layer run, between QKV and O."""
    cfg = configs.config(name)
    m, keep = fake_model(cfg, preset)
    m.cfg.attention, m.cfg.max_pos, m.cfg.pos0 = 1, max_pos, 0
    recs = phase_table(m, B)
    S = cfg["n_codebooks"] - 1
    assert len(recs) == 5 * cfg["n_layers"] + 2 + S * (5 * cfg["d_layers"] + 1) + 1
    kinds = [r["kind"] for r in recs]
    assert kinds[:5] == [_lib.PHASE_GEMV, _lib.PHASE_ATTENTION] + [_lib.PHASE_GEMV] * 3
    assert kinds.count(_lib.PHASE_ATTENTION) == cfg["n_layers"] + S * cfg["d_layers"]
    assert violations(recs) == []
    # O waits for the attention step's output words
    o = recs[2]
    assert any(g["tagged"] and g["producer"] == 1 for g in o["inp"])


def test_validator_finds_planted_attention_mistakes():
    """The attention rules catch a table broken on purpose (on the host)."""
    import copy
    cfg = configs.config("frame-small")
    m, keep = fake_model(cfg, "A")
    m.cfg.attention, m.cfg.max_pos, m.cfg.pos0 = 1, 300, 0
    recs = phase_table(m, 2)
    assert violations(recs) == []
    att = [i for i, r in enumerate(recs) if r["kind"] == _lib.PHASE_ATTENTION]
    depth = [i for i in att if i > 5 * cfg["n_layers"]]
    # a depth attention step that no longer waits for its QKV: what the layer's
    # earlier steps wrote into the cache is then read without an ordering
    r1 = copy.deepcopy(recs)
    j = depth[cfg["d_layers"]]           # the first layer at the second codebook step
    for g in r1[j]["inp"]:
        if g["tagged"]:
            g["tagged"] = False
    assert violations(r1)
    # a GEMV reading a KV cache that an attention step writes
    r2 = copy.deepcopy(recs)
    cache = copy.deepcopy(next(g for g in recs[att[0]]["out"] if not g["tagged"]))
    r2[att[0] + 1]["inp"].append(cache)
    assert violations(r2)
    # O reading the attention output as if the QKV GEMV had written it
    r3 = copy.deepcopy(recs)
    g = next(g for g in r3[att[0] + 1]["inp"] if g["tagged"] and g["producer"] == att[0])
    g["producer"] = att[0] - 1
    assert violations(r3)


def test_validator_finds_planted_mistakes():
    """Each rule catches a table broken on purpose (on the host)."""
    cfg = configs.config("frame-small")
    m, keep = fake_model(cfg, "A")
    recs = phase_table(m, 2)
    assert violations(recs) == []
    import copy
    # a consumer waiting for the wrong producer
    r1 = copy.deepcopy(recs)
    g = next(g for g in r1[5]["inp"] if g["tagged"])
    g["producer"] -= 1
    assert violations(r1)
    # a step writing what an earlier step wrote (the same slot twice in a frame)
    r2 = copy.deepcopy(recs)
    r2[9]["out"].append(copy.deepcopy(r2[4]["out"][0]))
    assert violations(r2)
    # an untagged read of a buffer a GEMV of the frame writes
    r3 = copy.deepcopy(recs)
    g = next(g for g in r3[6]["inp"] if g["tagged"])
    g["tagged"] = False
    assert violations(r3)
    # a wait for a later step
    r4 = copy.deepcopy(recs)
    g = next(g for g in r4[3]["inp"] if g["tagged"])
    g["producer"] = 7
    assert violations(r4)


GUIDED_CASES = [("frame-small", "A", 2, 0, False), ("frame-small", "B", 6, 40, False),
                ("frame-small", "A", 4, 300, True), ("frame-full", "A", 2, 2048, True),
                ("frame-full", "C", 6, 0, True)]


@pytest.mark.parametrize("name,preset,B,max_pos,end", GUIDED_CASES)
def test_phase_table_ordering_with_the_guided_draw(name, preset, B, max_pos, end):
    """The reference's draw: a draw step after the lm_head and after each
    head, which the next step's gather and the frame end read (with and
    without decode attention and the end token)."""
    cfg = configs.config(name)
    m, keep = fake_model(cfg, preset)
    m.cfg.top_k, m.cfg.cfg_scale = 50, 1.5
    if end:
        m.cfg.end_id = cfg["end_token"]
    if max_pos:
        m.cfg.attention, m.cfg.max_pos, m.cfg.pos0 = 1, max_pos, 0
    recs = phase_table(m, B)
    S = cfg["n_codebooks"] - 1
    per = 5 if max_pos else 4
    assert len(recs) == per * cfg["n_layers"] + 2 + S * (per * cfg["d_layers"] + 1) + S + 1 + 1
    kinds = [r["kind"] for r in recs]
    assert kinds.count(_lib.PHASE_DRAW) == S + 1
    lm = per * cfg["n_layers"]
    assert kinds[lm] == _lib.PHASE_GEMV and kinds[lm + 1] == _lib.PHASE_DRAW
    assert violations(recs) == []
    # the depth input's gather reads the draw's winner records, tagged by it
    assert any(g["tagged"] and g["producer"] == lm + 1 for g in recs[lm + 3]["inp"])
    # a draw that reads logits an earlier step wrote breaks rule (6)
    import copy
    r1 = copy.deepcopy(recs)
    r1[lm + 1]["inp"][0]["producer"] = lm - 1
    assert violations(r1)


def test_phase_table_refuses_what_the_persistent_frame_does_not_carry():
    cfg = configs.config("frame-small")
    m, keep = fake_model(cfg, "A")
    L = _lib.lib()
    assert L.m3_frame_phase_table(None, ctypes.c_void_p(STATE), 2, ctypes.c_void_p(CODES),
                                  None, 0) == _lib.M3_ERR_NULL
    n = L.m3_frame_phase_table(ctypes.byref(m), ctypes.c_void_p(STATE), 2, ctypes.c_void_p(CODES),
                               None, 0)
    recs = (_lib.PhaseRecord * (n - 1))()
    assert L.m3_frame_phase_table(ctypes.byref(m), ctypes.c_void_p(STATE), 2,
                                  ctypes.c_void_p(CODES), recs, n - 1) == _lib.M3_ERR_WORKSPACE
