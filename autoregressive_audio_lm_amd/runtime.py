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
                attention: int = 0, max_pos: int = 0, pos0: int = 0,
                end_token: bool = False) -> _lib.Config:
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
        top_k=int(top_k), attention=int(attention), max_pos=int(max_pos), pos0=int(pos0),
        end_id=int(cfg["end_token"]) if end_token else -1)


def frame_weight_bytes(c: _lib.Config) -> int:
    return int(lib().m3_frame_weight_bytes(ctypes.byref(c)))


class NoFramesError(RuntimeError):
    """A song drew the end token at its first frame: nothing was generated."""


def frames_generated(stop, frame0: int):
    """From the rows' stop words (0, or 1 + the frame of the first end token):
    the frames each row generated before its end token, or -1 while it is
    still running.  A row whose end token came at its first frame (frame0)
    generated nothing, which stops the whole request (DiffSynth-Studio
    MiniMax-Music3 stage 2)."""
    import numpy as np
    stop = np.asarray(stop, np.int64)
    n = np.where(stop > 0, stop - 1 - int(frame0), -1)
    if np.any(n == 0):
        raise NoFramesError(f"rows {np.flatnonzero(n == 0).tolist()} drew the end token at "
                            f"their first frame")
    return n


class DecodeModel:
    """All weights of one decode frame, packed on the device.

    `md` is a model dict of device tensors (bf16 sources, fp32 gammas) as made
    by autoregressive_audio_lm_amd.synth.make_model(..., device="cuda").  With
    free_sources=True the bf16 sources of packed matrices are dropped after
    packing."""

    def __init__(self, md: dict, seed: int = 0, temperature: float = 1.0,
                 free_sources: bool = False, cfg_scale: float = 1.5, top_k: int = 0,
                 attention: int = 0, max_pos: int = 0, pos0: int = 0, end_token: bool = False):
        """end_token: the semantic draw also takes the end token (its lm_head
        row md["lm_end"] packed first), and frames set the rows' stop words."""
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
                                  cfg_scale, top_k, attention, max_pos, pos0, end_token)
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
                dst[-1]["q_norm"], dst[-1]["k_norm"] = self._keep[-2], self._keep[-1]
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
            lm_head=packed(torch.cat([md["lm_end"], md["lm_head"]], 0) if end_token
                           else md["lm_head"], self.fmt_lm),
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
        self.dm, self.B, self.frame0 = dm, B, int(frame0)
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
        """The body output: the residual stream after the last body layer."""
        return self.h_layers()[-1]

    def _slots(self, name: str, dtype: torch.dtype, shape: tuple) -> torch.Tensor:
        off = getattr(self.layout, name)
        n = 1
        for s in shape:
            n *= s
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.state[off:off + n * esz].view(dtype).view(*shape)

    # per-stage slots of the state (m3_frame_layout): name -> (tagged name, shape)
    def _slot_shapes(self) -> dict:
        c, B = self.dm.config, self.B
        L, S, DL = c.n_layers, c.n_codebooks - 1, c.d_layers
        nq = c.n_heads * c.head_dim
        nqkv = nq + 2 * c.n_kv_heads * c.head_dim
        dq = c.d_heads * c.d_head_dim
        return {"h": ("th", (L, B, c.hidden)), "qkv": ("tqkv", (L, B, nqkv)),
                "ho": ("th2", (L, B, c.hidden)), "mlp": ("tmlp", (L, B, c.ffn)),
                "ao": ("tao", (L, B, nq)), "u": ("tu", (B, c.d_hidden)),
                "hd": ("thd", (S, DL + 1, B, c.d_hidden)), "dqkv": ("tdqkv", (S, DL, B, 3 * dq)),
                "hdo": ("thd2", (S, DL, B, c.d_hidden)), "dmlp": ("tdmlp", (S, DL, B, c.d_ffn)),
                "dao": ("tdao", (S, DL, B, dq))}

    def slots(self, name: str, tagged: bool = False) -> torch.Tensor:
        """A per-stage stream of the last frame: body [n_layers, B, cols] for
        h (after each layer), qkv, ho (after O + residual), mlp (SwiGLU) and ao
        (attention output); u [B, d_hidden]; depth [steps, d_layers + 1, B, D]
        for hd (slot 0 the step input, slot l + 1 after depth layer l) and
        [steps, d_layers, B, cols] for dqkv, hdo, dmlp, dao.  bf16 after an
        eager or graph frame; tagged=True: the persistent frame's 32-bit words
        (bf16 value in the low 16 bits)."""
        tname, shape = self._slot_shapes()[name]
        if tagged:
            if tname is None:
                raise ValueError(f"{name} has no tagged form")
            return self._slots(tname, torch.int32, shape)
        return self._slots(name, torch.bfloat16, shape)

    def h_layers(self, tagged: bool = False) -> torch.Tensor:
        """[n_layers, B, hidden]: the residual stream after each body layer."""
        return self.slots("h", tagged)

    def depth_slots(self, tagged: bool = False) -> torch.Tensor:
        """[n_codebooks-1, d_layers+1, B, d_hidden]: each depth step's input
        and the residual stream after each of its layers."""
        return self.slots("hd", tagged)

    @property
    def dlogits(self) -> torch.Tensor:
        """[n_codebooks-1, B, code_vocab] fp32: each depth step's head logits."""
        c = self.dm.config
        return self._slots("dlogits", torch.float32, (c.n_codebooks - 1, self.B, c.code_vocab))

    @property
    def logits(self):
        """[B, n_slice] fp32 semantic logits ([B, 1 + n_slice] with the end
        token, column 0)."""
        c = self.dm.config
        n = c.n_slice + (1 if c.end_id >= 0 else 0)
        ld = (n + 7) // 8 * 8
        return self.view("logits", torch.float32, ld)[:, :n]

    def prefill(self, xp: torch.Tensor, stream=None, trace: bool = False):
        """The prompt before the first frame (attention = 1, bf16 body): rows
        xp [B, P, hidden] bf16 (row b's prompt embeddings, P = the config's
        pos0, so that frame 0 continues at position P) run through every body
        layer as the prompt prefill (m3_rmsnorm_rows, m3_prefill_gemm,
        m3_prefill_qk_norm_rope writing each layer's keys and values at
        positions 0 .. P-1 straight into this state's caches,
        m3_prefill_attention), so the frames attend over the prompt with no
        copy.  trace: return per layer the QKV, attention output, residual
        stream after O, SwiGLU output and residual stream after down
        ([B * P, *] host bf16 bits, rows ordered [b][t]; the launches go to
        the current stream then)."""
        c, B = self.dm.config, self.B
        if not c.attention:
            raise ValueError("prefill fills the caches of an attention frame state")
        if self.dm.fmt_body != m3.BF16:
            raise ValueError("the prompt prefill GEMM takes bf16 body weights")
        if xp.dim() != 3 or xp.shape[0] != B or xp.shape[2] != c.hidden or xp.shape[1] != c.pos0:
            raise ValueError(f"prompt rows must be [B, pos0={c.pos0}, hidden]")
        P, H, F = xp.shape[1], c.hidden, c.ffn
        nq, nkv = c.n_heads * 128, c.n_kv_heads * 128
        dev = self.state.device
        h = xp.reshape(B * P, H).contiguous().clone()
        a = torch.empty(B * P, H, dtype=torch.bfloat16, device=dev)
        qkv = torch.empty(B * P, nq + 2 * nkv, dtype=torch.bfloat16, device=dev)
        att = torch.empty(B * P, nq, dtype=torch.bfloat16, device=dev)
        mlp = torch.empty(B * P, F, dtype=torch.bfloat16, device=dev)
        rope = self.view("rope", torch.float32, 128, rows=max(c.max_pos, 8))
        n = B * c.n_kv_heads * c.max_pos * 128
        kall = self.state[self.layout.kcache:self.layout.kcache + 2 * n * c.n_layers]
        vall = self.state[self.layout.vcache:self.layout.vcache + 2 * n * c.n_layers]
        out = []
        for l, W in enumerate(self.dm.packed_layers):
            kc = kall[2 * n * l:2 * n * (l + 1)].view(torch.bfloat16).view(B, c.n_kv_heads, c.max_pos, 128)
            vc = vall[2 * n * l:2 * n * (l + 1)].view(torch.bfloat16).view(B, c.n_kv_heads, c.max_pos, 128)
            m3.rmsnorm_rows(h, W["attn_norm"], c.eps, a=a, stream=stream)
            m3.prefill_gemm(W["qkv"], nq + 2 * nkv, H, a, y=qkv, stream=stream)
            q = m3.prefill_qk_norm_rope(qkv, B, c.n_heads, c.n_kv_heads, W["q_norm"], W["k_norm"],
                                        rope, 0, kc, vc, eps=c.eps, stream=stream)
            m3.prefill_attention(q, B, c.n_heads, c.n_kv_heads, kc, vc, 0, out=att, stream=stream)
            ho = m3.prefill_gemm(W["o"], H, nq, att, epi=m3.EPI_RESIDUAL, residual=h, stream=stream)
            m3.rmsnorm_rows(ho, W["ffn_norm"], c.eps, a=a, stream=stream)
            m3.prefill_gemm(W["gate_up"], 2 * F, H, a, y=mlp, epi=m3.EPI_SWIGLU, stream=stream)
            h = m3.prefill_gemm(W["down"], H, F, mlp, epi=m3.EPI_RESIDUAL, residual=ho, stream=stream)
            if trace:
                from . import synth
                out.append({k: synth.bits(v) for k, v in
                            (("qkv", qkv), ("ao", att), ("ho", ho), ("mlp", mlp), ("h", h))})
        return out if trace else None

    def poll_stop(self):
        """The host's read of the stop words (every 16 frames, alongside the
        code ring): frames_generated for each row."""
        return frames_generated(self.stop.cpu().numpy(), self.frame0)

    @property
    def stop(self) -> torch.Tensor:
        """[B] int32 stop words: 0, or 1 + the frame that drew the end token."""
        return self.view("stop", torch.int32, 1).view(self.B)

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

    def capture(self, stream, depth_only: bool = False) -> None:
        """Capture one frame into a HIP graph on `stream` (not the default
        stream); depth_only: the depth decoder's part of the frame alone
        (m3_depth_graph_create), reading the body output and semantic draw of
        the state's last whole frame."""
        g = ctypes.c_void_p()
        create = lib().m3_depth_graph_create if depth_only else lib().m3_frame_graph_create
        check(create(ctypes.byref(self.dm.model), ctypes.c_void_p(self.state.data_ptr()), self.B,
                     ctypes.c_void_p(self.codes.data_ptr()), ctypes.c_void_p(stream.cuda_stream),
                     ctypes.byref(g)))
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

    def persistent_clock(self, on: bool = True) -> None:
        """Attach (on) or detach the phase clock of the persistent frame
        (m3_frame_persistent_clock): later launches record per workgroup the
        real-time counter at each phase's entry, operand staged and end."""
        if not on:
            check(lib().m3_frame_persistent_clock(self.persistent, None, 0, None, None))
            self._clk = None
            return
        nb = int(lib().m3_frame_persistent_clock_bytes(self.persistent))
        self._clk = torch.zeros(nb // 8, dtype=torch.int64, device=self.state.device)
        nph, nwg = ctypes.c_int(), ctypes.c_int()
        check(lib().m3_frame_persistent_clock(self.persistent, ctypes.c_void_p(self._clk.data_ptr()),
                                              nb, ctypes.byref(nph), ctypes.byref(nwg)))
        self._clk_dims = (nph.value, nwg.value)

    def phase_clock(self):
        """The last launch's phase clock as an int64 array [3, n_phases,
        n_workgroups] (slots: entry, operand staged, end; 0 = not written)."""
        nph, nwg = self._clk_dims
        return self._clk.view(3, nph, nwg).cpu().numpy()

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
