"""Decode-frame runtime: packs a model's weights on the GPU, owns the frame
state, and drives m3_decode_frame_weights (eagerly or as a replayed HIP
graph).  Marshalling only; all compute is in libm3."""
from __future__ import annotations

import ctypes

import torch

from . import _lib, m3
from ._lib import check, lib


def make_config(cfg: dict, fmt_body: int, fmt_lm: int, fmt_depth: int, seed: int = 0,
                temperature: float = 1.0, cfg_scale: float = 1.5, top_k: int = 0,
                attention: int = 0, max_pos: int = 0, pos0: int = 0) -> _lib.Config:
    """top_k == 0: one draw per row; top_k > 0: the reference's draw over
    (conditional, unconditional) row pairs with guidance cfg_scale.
    attention == 0: the identity stub; 1: decode attention over caches of
    max_pos positions, frame f at position pos0 + f."""
    return _lib.Config(
        hidden=cfg["H"], n_layers=cfg["n_layers"], n_heads=cfg["n_heads"],
        n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], ffn=cfg["F"],
        vocab_base=cfg["vocab_base"], n_slice=cfg["V0"], d_hidden=cfg["D"],
        d_layers=cfg["d_layers"], d_heads=cfg["d_heads"], d_head_dim=cfg["d_head_dim"],
        d_ffn=cfg["Fd"], n_codebooks=cfg["n_codebooks"], code_vocab=cfg["code_vocab"],
        fmt_body=fmt_body, fmt_lm=fmt_lm, fmt_depth=fmt_depth, eps=float(cfg["eps"]),
        temperature=float(temperature), seed=int(seed), cfg_scale=float(cfg_scale),
        top_k=int(top_k), attention=int(attention), max_pos=int(max_pos), pos0=int(pos0))


def frame_weight_bytes(c: _lib.Config) -> int:
    return int(lib().m3_frame_weight_bytes(ctypes.byref(c)))


class DecodeModel:
    """All weights of one decode frame, packed on the device.

    `md` is a model dict of device tensors (bf16 sources, fp32 gammas) as made
    by autoregressive_audio_lm_amd.synth.make_model(..., device="cuda").  With
    free_sources=True the bf16 sources of packed matrices are dropped after
    packing."""

    def __init__(self, md: dict, seed: int = 0, temperature: float = 1.0,
                 free_sources: bool = False, cfg_scale: float = 1.5, top_k: int = 0,
                 attention: int = 0, max_pos: int = 0, pos0: int = 0):
        cfg = md["cfg"]
        # the C side reads host arrays of these lengths from the config
        nsteps = cfg["n_codebooks"] - 1
        if (len(md["layers"]) != cfg["n_layers"] or len(md["d_layers"]) != cfg["d_layers"]
                or len(md["heads"]) != nsteps or len(md["audio_emb"]) != nsteps
                or len(md["emb"]) != max(nsteps - 1, 0)):
            raise ValueError("model arrays do not match the config's layer and codebook counts")
        self.cfg_dict = cfg
        self.fmt_body, self.fmt_lm, self.fmt_depth = md["fmt_body"], md["fmt_lm"], md["fmt_depth"]
        self.config = make_config(cfg, self.fmt_body, self.fmt_lm, self.fmt_depth, seed, temperature,
                                  cfg_scale, top_k, attention, max_pos, pos0)
        self._keep = []

        def keep(t):
            t = t.contiguous()
            self._keep.append(t)
            return ctypes.c_void_p(t.data_ptr())

        def packed(W, fmt, flags=0):
            P = m3.pack(fmt, W.contiguous(), flags)
            self._keep.append(P)
            return ctypes.c_void_p(P.data_ptr())

        self.packed_layers, self.packed_dlayers = [], []

        def layer(L, fmt, dst):
            gu = torch.cat([L["gate"], L["up"]], 0)
            lw = _lib.LayerWeights(packed(L["qkv"], fmt), packed(L["o"], fmt),
                                   packed(gu, fmt, m3.PACK_GLU_INTERLEAVE), packed(L["down"], fmt),
                                   keep(L["attn_norm"]), keep(L["ffn_norm"]))
            # the four packed tensors just appended, the two gammas after them
            dst.append(dict(zip(("qkv", "o", "gate_up", "down", "attn_norm", "ffn_norm"),
                                self._keep[-6:])))
            if "q_norm" in L:                # per-head q/k norms (decode attention)
                lw.q_norm, lw.k_norm = keep(L["q_norm"]), keep(L["k_norm"])
            del gu
            if free_sources:
                for k in ("qkv", "o", "gate", "up", "down"):
                    L[k] = None
            return lw

        nl = len(md["layers"])
        self._layers = (_lib.LayerWeights * nl)(
            *[layer(L, self.fmt_body, self.packed_layers) for L in md["layers"]])
        self._dlayers = (_lib.LayerWeights * len(md["d_layers"]))(
            *[layer(L, self.fmt_depth, self.packed_dlayers) for L in md["d_layers"]])
        heads = [packed(W, self.fmt_depth) for W in md["heads"]]
        self._heads = (ctypes.c_void_p * len(heads))(*heads)
        embs = [keep(e) for e in md["emb"]]
        self._emb = (ctypes.c_void_p * max(len(embs), 1))(*embs)
        aembs = [keep(e) for e in md["audio_emb"]]
        self._aemb = (ctypes.c_void_p * len(aembs))(*aembs)
        self.model = _lib.Model(
            cfg=self.config,
            layers=ctypes.cast(self._layers, ctypes.c_void_p),
            final_norm=keep(md["final_norm"]),
            lm_head=packed(md["lm_head"], self.fmt_lm),
            p_in=packed(md["p_in"], self.fmt_depth),
            emb1=keep(md["emb1"]),
            emb=ctypes.cast(self._emb, ctypes.c_void_p),
            d_layers_w=ctypes.cast(self._dlayers, ctypes.c_void_p),
            d_final_norm=keep(md["d_final_norm"]),
            heads=ctypes.cast(self._heads, ctypes.c_void_p),
            tok_emb_audio=keep(md["tok_emb_audio"]),
            audio_emb=ctypes.cast(self._aemb, ctypes.c_void_p))
        if free_sources:
            md["lm_head"] = md["p_in"] = None
            md["heads"] = []

    def weight_bytes(self) -> int:
        return frame_weight_bytes(self.config)

    def set_draw(self, cfg_scale: float = 1.5, top_k: int = 0) -> None:
        """Switch the frame's draws (per row, or with top_k > 0 the
        reference's draw over row pairs) for frame states made from now on;
        the packed weights are shared."""
        for c in (self.config, self.model.cfg):
            c.cfg_scale = float(cfg_scale)
            c.top_k = int(top_k)

    def set_attention(self, attention: int = 1, max_pos: int = 2048, pos0: int = 0) -> None:
        """Switch the frame states made from now on between the identity stub
        (attention 0) and decode attention over caches of max_pos positions,
        frame f at position pos0 + f (attention 1); the packed weights are
        shared."""
        for c in (self.config, self.model.cfg):
            c.attention, c.max_pos, c.pos0 = int(attention), int(max_pos), int(pos0)


class FrameState:
    """Caller-owned frame state (device) for B lockstep rows, plus the [B, 8]
    code output of the last frame."""

    def __init__(self, dm: DecodeModel, B: int, x0: torch.Tensor, frame0: int = 0, stream=None):
        self.dm, self.B = dm, B
        self.layout = _lib.FrameLayout()
        check(lib().m3_frame_layout_get(ctypes.byref(dm.config), B, ctypes.byref(self.layout)))
        dev = x0.device
        self.buf = torch.empty(self.layout.total + 256, dtype=torch.uint8, device=dev)
        off = (-self.buf.data_ptr()) % 256
        self.state = self.buf[off:off + self.layout.total]
        self.codes = torch.zeros(B, 8, dtype=torch.int32, device=dev)
        self.graph = None
        self.persistent = None
        check(lib().m3_frame_state_init(ctypes.byref(dm.config), B, ctypes.c_void_p(self.state.data_ptr()),
                                        ctypes.c_void_p(x0.contiguous().data_ptr()), int(frame0),
                                        m3._stream(stream)))

    def view(self, name: str, dtype: torch.dtype, cols: int, rows: int | None = None) -> torch.Tensor:
        off = getattr(self.layout, name)
        rows = self.B if rows is None else rows
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.state[off:off + rows * cols * esz].view(dtype).view(rows, cols)

    @property
    def x(self):
        return self.view("x", torch.bfloat16, self.dm.config.hidden)

    @property
    def h(self):
        return self.view("h", torch.bfloat16, self.dm.config.hidden)

    @property
    def logits(self):
        return self.view("logits", torch.float32, self.dm.config.n_slice)

    @property
    def frame(self) -> torch.Tensor:
        return self.state[self.layout.frame:self.layout.frame + 4].view(torch.int32)

    @property
    def ring(self):
        return self.view("ring", torch.int32, self.B * 8, rows=16).view(16, self.B, 8)

    def decode(self, stream=None) -> int:
        nbytes = ctypes.c_uint64(0)
        check(lib().m3_decode_frame_weights(ctypes.byref(self.dm.model),
                                            ctypes.c_void_p(self.state.data_ptr()), self.B,
                                            ctypes.c_void_p(self.codes.data_ptr()),
                                            ctypes.byref(nbytes), m3._stream(stream)))
        return int(nbytes.value)

    def capture(self, stream) -> None:
        """Capture one frame into a HIP graph on `stream` (not the default stream)."""
        g = ctypes.c_void_p()
        check(lib().m3_frame_graph_create(ctypes.byref(self.dm.model),
                                          ctypes.c_void_p(self.state.data_ptr()), self.B,
                                          ctypes.c_void_p(self.codes.data_ptr()),
                                          ctypes.c_void_p(stream.cuda_stream), ctypes.byref(g)))
        self.graph = g

    def replay(self, stream) -> None:
        check(lib().m3_frame_graph_launch(self.graph, ctypes.c_void_p(stream.cuda_stream)))

    def persistent_create(self, stream=None) -> None:
        """Record the frame as the phase table of one persistent launch."""
        h = ctypes.c_void_p()
        check(lib().m3_frame_persistent_create(ctypes.byref(self.dm.model),
                                               ctypes.c_void_p(self.state.data_ptr()), self.B,
                                               ctypes.c_void_p(self.codes.data_ptr()),
                                               m3._stream(stream), ctypes.byref(h)))
        self.persistent = h

    def persistent_launch(self, stream=None) -> None:
        check(lib().m3_frame_persistent_launch(self.persistent, m3._stream(stream)))

    @property
    def err(self) -> torch.Tensor:
        """Nonzero once a persistent frame gave up waiting (its outputs are
        invalid), or with M3_ERR_ATTN_FULL set once an attention frame's
        position reached max_pos."""
        return self.state[self.layout.err:self.layout.err + 4].view(torch.int32)

    def release(self) -> None:
        if self.graph is not None:
            check(lib().m3_frame_graph_destroy(self.graph))
            self.graph = None
        if getattr(self, "persistent", None) is not None:
            check(lib().m3_frame_persistent_destroy(self.persistent))
            self.persistent = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass
