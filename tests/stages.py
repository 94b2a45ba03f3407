"""Operation-by-operation (teacher-forced) checks of one decode frame against
the oracle (imported by tests only).

TensorFold PR #987 (summary) checks its engine for parity at every stage,
teacher-forced: each stage is given the same input on both sides and only
its own output is compared, so a stage is judged by its own rounding, not by
how earlier differences grew along the chain.  The frame state keeps the
output of every operation of a frame (include/m3.h, m3_frame_layout), and
each is compared with the oracle's operation applied to the GPU's own input
of that operation, at that operation's tolerance (tests/parity.py):

* per body layer and per depth layer of every codebook step:
  - QKV = W_qkv . rmsnorm(h_in)          -> check_bf16 (bf16 GEMV output)
  - the stream after O: bf16(h_in + bf16(W_o . v))  -> check_residual,
    v the identity stub's V heads of the GPU's QKV (or, with decode
    attention, the GPU's attention output, itself checked against the
    oracle's q/k norm + RoPE + attention of the GPU's QKV over the cache)
  - SwiGLU of W_gu . rmsnorm(stream after O)        -> check_swiglu
  - the stream after down: bf16(after O + bf16(W_down . m)) -> check_residual
* the lm_head logits (fp32) and the depth input projection u (bf16) from the
  final norm of the GPU's body output; each depth head's logits (fp32) from
  the final norm of the GPU's step output;
* every draw: the oracle sampler on the GPU's own fp32 logits, bit-exact;
* each depth step's input bf16(u + Emb_j[c_{j-1}]) from the GPU's u and
  codes, bit-exact (one rounding of an exact sum);
* the next frame's input from the GPU's codes (float32 sum of 8 bf16 rows on
  the GPU, float64 in the oracle; at most one ulp apart, 99.9% identical).
"""
from __future__ import annotations

import numpy as np

import oracle as O
import parity as P


def untag(t) -> np.ndarray:
    """A persistent frame's tagged words -> bf16 bits (the low 16 bits)."""
    return (t.cpu().numpy().view(np.uint32) & 0xFFFF).astype(np.uint16)


def read_frame(st, tagged: bool) -> dict:
    """Every operation's output of the frame just run on FrameState st."""
    from autoregressive_audio_lm_amd import synth
    rd = untag if tagged else synth.bits
    got = {k: rd(st.slots(k, tagged)) for k in ("h", "qkv", "ho", "mlp", "u", "hd", "dqkv", "hdo",
                                                 "dmlp")}
    if st.dm.config.attention:
        got["ao"] = rd(st.slots("ao", tagged))
        got["dao"] = rd(st.slots("dao", tagged))
    got.update(logits=st.logits.cpu().numpy(), dlogits=st.dlogits.cpu().numpy(),
               codes=st.codes.cpu().numpy(), x=synth.bits(st.x))
    return got


def read_caches(st) -> dict:
    """Host copies of the frame state's KV caches (attention = 1): body
    [n_layers][B, n_kv, max_pos, 128] and depth [d_layers][B, d_heads, 8, 128]."""
    import torch
    from autoregressive_audio_lm_amd import synth
    c, B = st.dm.config, st.B
    out = {}
    for name, L, nh, mp in (("kcache", c.n_layers, c.n_kv_heads, c.max_pos),
                            ("vcache", c.n_layers, c.n_kv_heads, c.max_pos),
                            ("dkcache", c.d_layers, c.d_heads, 8), ("dvcache", c.d_layers, c.d_heads, 8)):
        off, n = getattr(st.layout, name), L * B * nh * mp * 128
        out[name] = synth.bits(st.state[off:off + 2 * n].view(torch.bfloat16).view(L, B, nh, mp, 128))
    return out


class Stats:
    """Identical fraction (against the oracle's own bf16 rounding) and worst
    |deviation| / rms per checked bf16 output."""

    def __init__(self):
        self.rows = []

    def add(self, what, got_bits, want_exact):
        g = O.bf16_to_f64(got_bits)
        w = np.asarray(want_exact, np.float64)
        self.rows.append((what, float(np.mean(np.asarray(got_bits) == O.f64_to_bf16(w))),
                          float(np.max(np.abs(g - w) / P.row_rms(w)))))

    def summary(self) -> str:
        if not self.rows:
            return "nothing checked"
        worst = min(self.rows, key=lambda r: r[1])
        dev = max(self.rows, key=lambda r: r[2])
        return (f"{len(self.rows)} outputs: min identical {worst[1]:.5f} ({worst[0]}), "
                f"max |dev|/rms {dev[2]:.2e} ({dev[0]})")


def _op(what, fn, got, *args, **kw):
    try:
        fn(got, *args, **kw)
    except AssertionError as e:
        raise AssertionError(f"{what}: {e}") from None


def _layer(om, stats, kind, l, ln, pre, g, h_in, attn_step):
    """The four operations of one layer (kind "body" or "depth", layer l with
    weights dict ln) on the GPU's slots g = dict(qkv, ho, mlp, h_out)."""
    cfg = om.cfg
    eps = cfg["eps"]
    if kind == "body":
        nh, nkv = cfg["n_heads"], cfg["n_kv_heads"]
    else:
        nh = nkv = cfg["d_heads"]
    hd = 128
    M = lambda name: O.mat_of(om, kind, l, name)
    y = O.gemv(M("qkv"), O.rmsnorm(h_in, ln["attn_norm"], eps))
    stats.add(f"{pre} qkv", g["qkv"], y)
    _op(f"{pre} qkv", P.check_bf16, g["qkv"], y)
    if attn_step is None:
        o_in = O.attn_stub(g["qkv"], (nh + nkv) * hd, nh, nh // nkv, hd)
    else:
        o_in = attn_step(g["qkv"])
    y = O.gemv(M("o"), o_in)
    stats.add(f"{pre} after O", g["ho"], O.bf16_to_f64(h_in) + O.bf16_to_f64(O.f64_to_bf16(y)))
    _op(f"{pre} after O", P.check_residual, g["ho"], h_in, y)
    y = O.gemv(M("gu"), O.rmsnorm(g["ho"], ln["ffn_norm"], eps))
    _op(f"{pre} SwiGLU", P.check_swiglu, g["mlp"], y)
    y = O.gemv(M("down"), g["mlp"])
    stats.add(f"{pre} after down", g["h_out"],
              O.bf16_to_f64(g["ho"]) + O.bf16_to_f64(O.f64_to_bf16(y)))
    _op(f"{pre} after down", P.check_residual, g["h_out"], g["ho"], y)


def check_frame(om, got, x0, seed, frame, body_layers=None, depth_steps=None, rows=None,
                attn=None) -> Stats:
    """Compare every operation's output in `got` (read_frame) with the oracle
    on the GPU's own input of that operation.  body_layers / depth_steps: the
    layers and steps whose operations are checked (all by default); rows: the
    batch rows whose GEMV outputs are checked (all by default; a row's outputs
    depend on that row only, on both sides).  The draws, the step inputs and
    the feedback are always checked on every row.

    attn (frames with decode attention): dict(pos=the body position of the
    frame, before=read_caches() before the frame, after=read_caches() after
    it).  Each body layer's attention output is checked against the oracle's
    q/k norm + RoPE + attention of the GPU's QKV over the cache as it was
    before the frame plus the slot the oracle writes at pos (the GPU's written
    slot compared too); each depth layer's over the GPU's slots of the frame's
    earlier codebook positions plus its own at j - 1."""
    md, cfg = om.md, om.cfg
    eps, base, V0 = cfg["eps"], cfg["vocab_base"], cfg["V0"]
    nL, dl = cfg["n_layers"], cfg["d_layers"]
    stats = Stats()
    codes = got["codes"]
    sub = got
    rsel = slice(None)
    if rows is not None:
        rsel = np.asarray(rows)
        sub = {}
        for k, v in got.items():
            if k in ("h", "qkv", "ho", "mlp", "ao", "dlogits"):
                sub[k] = v[:, rsel]
            elif k in ("hd", "dqkv", "hdo", "dmlp", "dao"):
                sub[k] = v[:, :, rsel]
            else:
                sub[k] = v[rsel]
    x0s = np.asarray(x0)[rsel]

    def attn_step(cache, pos, n_q, n_kv, ln, ao_gpu, what):
        def step(qkv_gpu):
            kc, vc = cache
            q = O.qk_norm_rope(qkv_gpu, n_q, n_kv, ln["q_norm"], ln["k_norm"], eps, om._rope, pos,
                               kc, vc)
            o = O.decode_attention(q, kc, vc, pos + 1, n_q, n_kv)
            # q/k norm + RoPE + attention from the same QKV: q rounds once on
            # each side, as the decode-attention tests allow for
            _op(what, P.check_bf16_vs_bf16, ao_gpu, o, agree=0.97, rel=1e-2, width=128)
            return ao_gpu
        return step

    for l in (range(nL) if body_layers is None else body_layers):
        h_in = x0s if l == 0 else sub["h"][l - 1]
        g = dict(qkv=sub["qkv"][l], ho=sub["ho"][l], mlp=sub["mlp"][l], h_out=sub["h"][l])
        step = None
        if attn is not None:
            p = attn["pos"]
            kc = np.ascontiguousarray(attn["before"]["kcache"][l][rsel])
            vc = np.ascontiguousarray(attn["before"]["vcache"][l][rsel])
            step = attn_step((kc, vc), p, cfg["n_heads"], cfg["n_kv_heads"], md["layers"][l],
                             sub["ao"][l], f"body layer {l} attention")
        _layer(om, stats, "body", l, md["layers"][l], f"body layer {l}", g, h_in, step)
        if attn is not None:
            # the slots this frame wrote: k after norm + RoPE, v as computed
            for name, c_or in (("kcache", kc), ("vcache", vc)):
                _op(f"body layer {l} {name} slot {p}", P.check_bf16_vs_bf16,
                    attn["after"][name][l][rsel][:, :, p], c_or[:, :, p], width=128)
    a = O.rmsnorm(sub["h"][nL - 1], md["final_norm"], eps)
    _op("lm_head logits", P.check_f32, sub["logits"], O.gemv(O.mat_of(om, "lm_head"), a))
    _op("depth input projection", P.check_bf16, sub["u"], O.gemv(O.mat_of(om, "p_in"), a))

    def draw(lg, j, base, valid):
        # per-row Gumbel-argmax, or the reference's draw over row pairs
        if om.m.top_k > 0:
            return O.cfg_topk_draw(lg, scale=om.m.cfg_scale, top_k=om.m.top_k, seed=seed,
                                   frame=frame, draw=j, index_base=base, valid=valid)
        return O.gumbel_argmax(lg, seed=seed, frame=frame, draw=j, index_base=base, valid=valid)

    if om.m.end_id >= 0:
        # column 0 is the end token, column 1 + i code i
        ids = np.concatenate([[om.m.end_id], base + np.arange(V0)]).astype(np.int32)
        c0 = (O.cfg_topk_draw(got["logits"], scale=om.m.cfg_scale, top_k=om.m.top_k, seed=seed,
                              frame=frame, draw=0, ids=ids)
              if om.m.top_k > 0 else
              O.gumbel_argmax(got["logits"], seed=seed, frame=frame, draw=0, ids=ids))
    else:
        c0 = draw(got["logits"], 0, base, (base, base + V0))
    assert np.array_equal(c0, codes[:, 0]), ("draw 0", c0, codes[:, 0])
    for j in range(1, cfg["n_codebooks"]):
        d_in = O.step_input(om, j, codes, got["u"])
        assert np.array_equal(got["hd"][j - 1, 0], d_in), f"depth step {j} input"
        if depth_steps is None or j in depth_steps:
            for l in range(dl):
                g = dict(qkv=sub["dqkv"][j - 1, l], ho=sub["hdo"][j - 1, l],
                         mlp=sub["dmlp"][j - 1, l], h_out=sub["hd"][j - 1, l + 1])
                step = None
                if attn is not None:
                    cache = (np.ascontiguousarray(attn["after"]["dkcache"][l][rsel]),
                             np.ascontiguousarray(attn["after"]["dvcache"][l][rsel]))
                    step = attn_step(cache, j - 1, cfg["d_heads"], cfg["d_heads"],
                                     md["d_layers"][l], sub["dao"][j - 1, l],
                                     f"depth step {j} layer {l} attention")
                _layer(om, stats, "depth", l, md["d_layers"][l], f"depth step {j} layer {l}", g,
                       sub["hd"][j - 1, l], step)
        ad = O.rmsnorm(sub["hd"][j - 1, dl], md["d_final_norm"], eps)
        _op(f"depth head {j} logits", P.check_f32, sub["dlogits"][j - 1],
            O.gemv(O.mat_of(om, "head", j), ad))
        cj = draw(got["dlogits"][j - 1], j, 0, (0, 0))
        assert np.array_equal(cj, codes[:, j]), (f"draw {j}", cj, codes[:, j])
    want = O.feedback(om, codes)
    g, w = O.bf16_to_f64(got["x"]), O.bf16_to_f64(want)
    assert np.all(np.abs(g - w) <= 2 * P.half_ulp(w) * (1 + 1e-9)), "feedback"
    assert np.mean(got["x"] == want) >= 0.999, "feedback"
    return stats
