"""CPU oracle for the per-frame AR decode hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
``autoregressive_audio_lm_amd`` never imports it, and it never imports the
product package: the two share no code.

The arithmetic lives in ``m3_oracle.c`` (plain scalar C, float64 sums; the
sampler in fixed-sequence fp32), compiled with gcc into ``liboracle.so``.
This module is argument marshalling (numpy <-> C) plus a few plain-Python
definitions that are easier to read here (the weight-byte formula).

Definitions follow the pages (cited by title and section in the C source):
TensorFold PR #987 (Metal port) precision list and "What it adds";
diffusers issue #14486 item 3 and 4; the DiffSynth-Studio MiniMax-Music3
article, model overview and stage 2.

Parity status: every exported function is pinned by a CPU test against
something other than itself (see tests/test_oracle_*.py).  The depth-decoder
coupling inside ``decode_frame`` (how the body state enters the depth
decoder, which embedding each codebook step reads) is not given by the pages:
"parity unpinned" for that coupling; its components are pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, I8ROW, I8G128, FP8ROW = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH, _SRC, "-lm"]
        subprocess.check_call(cmd)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


# ---------------------------------------------------------------- ctypes ---
_P = ctypes.c_void_p


class Mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("w", _P), ("q", _P), ("s", _P)]


class SampleParams(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("frame", ctypes.c_uint32),
                ("draw", ctypes.c_uint32), ("temperature", ctypes.c_float),
                ("index_base", ctypes.c_int32), ("ids", _P),
                ("valid_lo", ctypes.c_int32), ("valid_hi", ctypes.c_int32),
                ("noise_override", _P)]


class Layer(ctypes.Structure):
    _fields_ = [("qkv", Mat), ("o", Mat), ("gu", Mat), ("down", Mat),
                ("attn_norm", _P), ("ffn_norm", _P), ("q_norm", _P), ("k_norm", _P)]


class Model(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int), ("n_layers", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("F", ctypes.c_int),
                ("layers", _P), ("final_norm", _P), ("lm_head", Mat),
                ("vocab_base", ctypes.c_int32), ("V0", ctypes.c_int),
                ("D", ctypes.c_int), ("d_layers", ctypes.c_int), ("d_heads", ctypes.c_int),
                ("d_head_dim", ctypes.c_int), ("Fd", ctypes.c_int),
                ("n_codebooks", ctypes.c_int), ("code_vocab", ctypes.c_int),
                ("p_in", Mat), ("emb1", _P), ("emb", _P), ("d_layers_w", _P),
                ("d_final_norm", _P), ("heads", _P), ("tok_emb_audio", _P),
                ("audio_emb", _P), ("eps", ctypes.c_float), ("cfg_scale", ctypes.c_float),
                ("top_k", ctypes.c_int), ("attention", ctypes.c_int), ("max_pos", ctypes.c_int),
                ("pos0", ctypes.c_int), ("rope", _P), ("kcache", _P), ("vcache", _P),
                ("dkcache", _P), ("dvcache", _P), ("end_id", ctypes.c_int32)]


class FrameTrace(ctypes.Structure):
    _fields_ = [("h_body", _P), ("logits0", _P), ("zgap", _P)]


def _declare(L):
    L.m3o_f64_to_bf16.restype = ctypes.c_uint16
    L.m3o_f64_to_bf16.argtypes = [ctypes.c_double]
    L.m3o_bf16_to_f64.restype = ctypes.c_double
    L.m3o_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.m3o_f64_to_bf16_n.argtypes = [_P, _P, ctypes.c_size_t]
    L.m3o_f32_to_bf16_n.argtypes = [_P, _P, ctypes.c_size_t]
    L.m3o_rmsnorm.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P,
                              ctypes.c_float, _P, ctypes.c_int]
    L.m3o_quant_i8row.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
    L.m3o_quant_i8g128.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
    L.m3o_gemv.argtypes = [ctypes.POINTER(Mat), _P, ctypes.c_int, ctypes.c_int, _P]
    L.m3o_gemv_rows.argtypes = [ctypes.POINTER(Mat), ctypes.c_int, ctypes.c_int, _P,
                                ctypes.c_int, ctypes.c_int, _P]
    L.m3o_swiglu_interleaved.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P]
    L.m3o_residual.argtypes = [_P, _P, ctypes.c_int, _P]
    L.m3o_rope_table.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, _P]
    L.m3o_qk_norm_rope.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, _P, _P, ctypes.c_float, _P, ctypes.c_int, _P,
                                   _P, _P, ctypes.c_int]
    L.m3o_decode_attention.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int, _P]
    L.m3o_attn_stub.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
    L.m3o_philox4x32_10.argtypes = [_P, _P, _P]
    L.m3o_logf.restype = ctypes.c_float
    L.m3o_logf.argtypes = [ctypes.c_float]
    L.m3o_uniform_from_word.restype = ctypes.c_float
    L.m3o_uniform_from_word.argtypes = [ctypes.c_uint32]
    L.m3o_gumbel.restype = ctypes.c_float
    L.m3o_gumbel.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                             ctypes.c_uint32, ctypes.c_uint32]
    L.m3o_gumbel_argmax.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(SampleParams), _P, _P, _P]
    L.m3o_fp8_decode.restype = ctypes.c_double
    L.m3o_fp8_decode.argtypes = [ctypes.c_uint8]
    L.m3o_fp8_encode.restype = ctypes.c_uint8
    L.m3o_fp8_encode.argtypes = [ctypes.c_double]
    L.m3o_quant_fp8row.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
    L.m3o_cfg_topk_draw.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_int, ctypes.POINTER(SampleParams), _P, _P,
                                    _P]
    L.m3o_decode_frame.argtypes = [ctypes.POINTER(Model), _P, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_float, _P, _P,
                                   ctypes.POINTER(FrameTrace)]
    L.m3o_num_threads.restype = ctypes.c_int
    L.m3o_layer_stub.argtypes = [ctypes.POINTER(Layer), _P, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_float]
    L.m3o_layer_attn.argtypes = [ctypes.POINTER(Layer), _P, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_float, _P, _P, _P, ctypes.c_int, ctypes.c_int]
    L.m3o_step_input.argtypes = [ctypes.POINTER(Model), ctypes.c_int, _P, _P, ctypes.c_int, _P]
    L.m3o_feedback.argtypes = [ctypes.POINTER(Model), _P, ctypes.c_int, _P]


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ bf16 ---
def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().m3o_f64_to_bf16_n(_ptr(v), _ptr(out), v.size)
    return out


def f32_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().m3o_f32_to_bf16_n(_ptr(v), _ptr(out), v.size)
    return out


# --------------------------------------------------------------- kernels ---
def rmsnorm(x, gamma, eps):
    """a = bf16(x * r * gamma), r = 1/sqrt(mean(x^2) + eps); gamma None -> x."""
    x = _c(x, np.uint16)
    B, K = x.shape
    a = np.empty_like(x)
    g = None if gamma is None else _c(gamma, np.float32)
    lib().m3o_rmsnorm(_ptr(x), B, K, K, _ptr(g), float(eps), _ptr(a), K)
    return a


def quant_i8row(W):
    W = _c(W, np.uint16)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    s = np.empty((N,), np.float32)
    lib().m3o_quant_i8row(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, s


def quant_i8g128(W):
    W = _c(W, np.uint16)
    N, K = W.shape
    assert K % 128 == 0
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // 128), np.float32)
    lib().m3o_quant_i8g128(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, s


def fp8_decode(c) -> float:
    return float(lib().m3o_fp8_decode(int(c) & 0xFF))


def fp8_encode(v) -> int:
    return int(lib().m3o_fp8_encode(float(v)))


def quant_fp8row(W):
    W = _c(W, np.uint16)
    N, K = W.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty((N,), np.float32)
    lib().m3o_quant_fp8row(_ptr(W), N, K, _ptr(q), _ptr(s))
    return q, s


class Matrix:
    """A weight matrix in one of the four formats, built from bf16 W by the
    oracle's own quantiser.  Keeps the numpy buffers alive for ctypes."""

    def __init__(self, W, fmt):
        W = _c(W, np.uint16)
        self.fmt, (self.N, self.K) = fmt, W.shape
        self.w = self.q = self.s = None
        if fmt == BF16:
            self.w = W
        elif fmt == I8ROW:
            self.q, self.s = quant_i8row(W)
        elif fmt == I8G128:
            self.q, self.s = quant_i8g128(W)
        elif fmt == FP8ROW:
            self.q, self.s = quant_fp8row(W)
        else:
            raise ValueError(fmt)

    def c(self) -> Mat:
        return Mat(self.fmt, self.N, self.K, _ptr(self.w), _ptr(self.q), _ptr(self.s))


def gemv(mat: Matrix, a, rows=None):
    """Exact (float64) y[b, n] = sum_k Wdeq[n, k] a[b, k]; rows=(row0, n) optional."""
    a = _c(a, np.uint16)
    B, K = a.shape
    assert K == mat.K
    cm = mat.c()
    if rows is None:
        y = np.empty((B, mat.N), np.float64)
        lib().m3o_gemv(ctypes.byref(cm), _ptr(a), B, K, _ptr(y))
    else:
        r0, nr = rows
        y = np.empty((B, nr), np.float64)
        lib().m3o_gemv_rows(ctypes.byref(cm), int(r0), int(nr), _ptr(a), B, K, _ptr(y))
    return y


def swiglu_interleaved(y):
    y = _c(y, np.float64)
    B, N2 = y.shape
    F = N2 // 2
    m = np.empty((B, F), np.uint16)
    lib().m3o_swiglu_interleaved(_ptr(y), B, F, _ptr(m))
    return m


def residual(y, h):
    y = _c(y, np.float64)
    h = _c(h, np.uint16)
    out = np.empty_like(h)
    lib().m3o_residual(_ptr(y), _ptr(h), h.size, _ptr(out))
    return out


def attn_stub(qkv, voff, n_heads, group, hd):
    qkv = _c(qkv, np.uint16)
    B, ldq = qkv.shape
    o = np.empty((B, n_heads * hd), np.uint16)
    lib().m3o_attn_stub(_ptr(qkv), B, ldq, int(voff), n_heads, group, hd, _ptr(o))
    return o


# ------------------------------------------------------ decode attention ---
def rope_table(max_pos, head_dim=128, theta=1e6):
    """[max_pos, head_dim/2, 2] fp32: cos, sin of p * theta^(-i/half), in float64."""
    t = np.empty((max_pos, head_dim // 2, 2), np.float32)
    lib().m3o_rope_table(int(max_pos), int(head_dim), float(theta), _ptr(t))
    return t


def qk_norm_rope(qkv, n_q, n_kv, q_gamma, k_gamma, eps, rope, pos, k_cache, v_cache, hd=128):
    """Per-head RMSNorm + RoPE of the q and k heads of qkv [B, ldq] at position
    pos; returns q [B, n_q*hd]; writes k and v into the caches (uint16 arrays
    [B, n_kv, max_pos, hd], modified in place)."""
    qkv = _c(qkv, np.uint16)
    B, ldq = qkv.shape
    assert k_cache.dtype == np.uint16 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.uint16 and v_cache.flags.c_contiguous
    max_pos = k_cache.shape[2]
    q = np.empty((B, n_q * hd), np.uint16)
    lib().m3o_qk_norm_rope(_ptr(qkv), B, ldq, int(n_q), int(n_kv), int(hd),
                           _ptr(_c(q_gamma, np.float32)), _ptr(_c(k_gamma, np.float32)),
                           float(eps), _ptr(_c(rope, np.float32)), int(pos), _ptr(q),
                           _ptr(k_cache), _ptr(v_cache), int(max_pos))
    return q


def decode_attention(q, k_cache, v_cache, T, n_q, n_kv, hd=128):
    """out [B, n_q*hd] bf16 = softmax(q k^T / sqrt(hd)) v over positions < T."""
    q = _c(q, np.uint16)
    B = q.shape[0]
    k_cache = _c(k_cache, np.uint16)
    v_cache = _c(v_cache, np.uint16)
    out = np.empty((B, n_q * hd), np.uint16)
    lib().m3o_decode_attention(_ptr(q), B, int(n_q), int(n_kv), int(hd), _ptr(k_cache),
                               _ptr(v_cache), int(k_cache.shape[2]), int(T), _ptr(out))
    return out


def interleave_gate_up(W_gate, W_up):
    """Rows 2i <- gate row i, 2i+1 <- up row i (the oracle's own arrangement)."""
    F, K = W_gate.shape
    out = np.empty((2 * F, K), np.uint16)
    out[0::2] = W_gate
    out[1::2] = W_up
    return out


# --------------------------------------------------------------- sampler ---
def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().m3o_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def logf(x: float) -> float:
    return float(np.float32(lib().m3o_logf(float(np.float32(x)))))


def uniform_from_word(w: int) -> float:
    return float(lib().m3o_uniform_from_word(int(w)))


def gumbel(seed, row, frame, draw, idx) -> np.float32:
    return np.float32(lib().m3o_gumbel(int(seed), int(row), int(frame), int(draw), int(idx)))


def gumbel_argmax(logits, seed=0, frame=0, draw=0, temperature=1.0, index_base=0,
                  ids=None, valid=(0, 0), noise=None, with_margin=False):
    lg = _c(logits, np.float32)
    B, V = lg.shape
    ids_a = None if ids is None else _c(ids, np.int32)
    nz = None if noise is None else _c(noise, np.float32)
    p = SampleParams(int(seed), int(frame), int(draw), float(temperature), int(index_base),
                     _ptr(ids_a), int(valid[0]), int(valid[1]), _ptr(nz))
    out = np.empty(B, np.int32)
    zb = np.empty(B, np.float32)
    z2 = np.empty(B, np.float32)
    lib().m3o_gumbel_argmax(_ptr(lg), B, V, V, ctypes.byref(p), _ptr(out), _ptr(zb), _ptr(z2))
    if with_margin:
        return out, zb, z2
    return out


def cfg_topk_draw(logits, scale=1.5, top_k=50, seed=0, frame=0, draw=0, temperature=1.0,
                  index_base=0, ids=None, valid=(0, 0), noise=None, with_kept=False,
                  with_gap=False):
    """The reference's draw over (conditional, unconditional) row pairs;
    logits [2S, V] -> ids [2S] (both rows of a song carry its draw)."""
    lg = _c(logits, np.float32)
    B, V = lg.shape
    if B % 2:
        raise ValueError("rows come in (conditional, unconditional) pairs")
    S = B // 2
    ids_a = None if ids is None else _c(ids, np.int32)
    nz = None if noise is None else _c(noise, np.float32)
    p = SampleParams(int(seed), int(frame), int(draw), float(temperature), int(index_base),
                     _ptr(ids_a), int(valid[0]), int(valid[1]), _ptr(nz))
    out = np.empty(B, np.int32)
    kept = np.empty(S, np.int32)
    gap = np.empty(S, np.float32)
    lib().m3o_cfg_topk_draw(_ptr(lg), S, V, V, float(scale), int(top_k), ctypes.byref(p),
                            _ptr(out), _ptr(kept), _ptr(gap))
    res = (out,) + ((kept,) if with_kept else ()) + ((gap,) if with_gap else ())
    return res[0] if len(res) == 1 else res


# ----------------------------------------------------------------- frame ---
class OracleModel:
    """Wraps a model dict (see autoregressive_audio_lm_amd.synth) into the C
    struct.  The oracle quantises int8 formats itself from the bf16 sources."""

    def __init__(self, md: dict, cfg_scale: float = 1.5, top_k: int = 0, attention: int = 0,
                 max_pos: int = 0, pos0: int = 0, end_token: bool = False):
        """top_k == 0: per-row draws; top_k > 0: the reference's draw over
        (conditional, unconditional) row pairs with guidance cfg_scale.
        attention == 1: decode attention over KV caches of max_pos positions
        (frame f at position pos0 + f); the caches are made zeroed for the
        batch size of the first frame (and again by reset_attention).
        end_token: the semantic draw also takes the end token, whose lm_head
        row is md["lm_end"] (m3o_decode_frame)."""
        self._keep = []
        self.md = md
        cfg = md["cfg"]
        fb, fl, fd = md["fmt_body"], md["fmt_lm"], md["fmt_depth"]

        self.mats = {}

        def mat(W, fmt, key=None):
            M = Matrix(W, fmt)
            self._keep.append(M)
            if key is not None:
                self.mats[key] = M
            return M.c()

        def keep(a, dt):
            a = _c(a, dt)
            self._keep.append(a)
            return a

        def layer(Ld, fmt, kind, i):
            gu = interleave_gate_up(Ld["gate"], Ld["up"])
            qn = _ptr(keep(Ld["q_norm"], np.float32)) if "q_norm" in Ld else None
            kn = _ptr(keep(Ld["k_norm"], np.float32)) if "k_norm" in Ld else None
            return Layer(mat(Ld["qkv"], fmt, (kind, i, "qkv")), mat(Ld["o"], fmt, (kind, i, "o")),
                         mat(gu, fmt, (kind, i, "gu")), mat(Ld["down"], fmt, (kind, i, "down")),
                         _ptr(keep(Ld["attn_norm"], np.float32)),
                         _ptr(keep(Ld["ffn_norm"], np.float32)), qn, kn)

        nl = len(md["layers"])
        LA = (Layer * max(nl, 1))(*[layer(L, fb, "body", i) for i, L in enumerate(md["layers"])])
        DL = (Layer * len(md["d_layers"]))(*[layer(L, fd, "depth", i)
                                            for i, L in enumerate(md["d_layers"])])
        heads = (Mat * len(md["heads"]))(*[mat(W, fd, ("head", j + 1))
                                           for j, W in enumerate(md["heads"])])
        embs = [keep(e, np.uint16) for e in md["emb"]]
        emb_arr = (ctypes.c_void_p * max(len(embs), 1))(*[e.ctypes.data for e in embs])
        aembs = [keep(e, np.uint16) for e in md["audio_emb"]]
        aemb_arr = (ctypes.c_void_p * len(aembs))(*[e.ctypes.data for e in aembs])
        self._keep += [LA, DL, heads, emb_arr, aemb_arr]
        self.cfg = cfg
        self.m = Model(
            cfg["H"], nl, cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["F"],
            ctypes.cast(LA, ctypes.c_void_p), _ptr(keep(md["final_norm"], np.float32)),
            mat(np.concatenate([md["lm_end"], md["lm_head"]], 0) if end_token else md["lm_head"],
                fl, ("lm_head", 0)), cfg["vocab_base"], cfg["V0"],
            cfg["D"], len(md["d_layers"]), cfg["d_heads"], cfg["d_head_dim"], cfg["Fd"],
            cfg["n_codebooks"], cfg["code_vocab"],
            mat(md["p_in"], fd, ("p_in", 0)), _ptr(keep(md["emb1"], np.uint16)),
            ctypes.cast(emb_arr, ctypes.c_void_p), ctypes.cast(DL, ctypes.c_void_p),
            _ptr(keep(md["d_final_norm"], np.float32)), ctypes.cast(heads, ctypes.c_void_p),
            _ptr(keep(md["tok_emb_audio"], np.uint16)), ctypes.cast(aemb_arr, ctypes.c_void_p),
            float(cfg["eps"]), float(cfg_scale), int(top_k), int(attention), int(max_pos),
            int(pos0))
        self.m.end_id = int(cfg["end_token"]) if end_token else -1
        self.cache_B = None
        if attention:
            self._rope = rope_table(max(max_pos, 8), cfg["head_dim"])
            self.m.rope = _ptr(self._rope)

    def reset_attention(self, B: int) -> None:
        """Fresh zeroed KV caches for B rows (attention mode)."""
        cfg, mp = self.cfg, self.m.max_pos
        self.kcache = [np.zeros((B, cfg["n_kv_heads"], mp, cfg["head_dim"]), np.uint16)
                       for _ in range(self.m.n_layers)]
        self.vcache = [np.zeros_like(c) for c in self.kcache]
        self.dkcache = [np.zeros((B, cfg["d_heads"], 8, cfg["d_head_dim"]), np.uint16)
                        for _ in range(self.m.d_layers)]
        self.dvcache = [np.zeros_like(c) for c in self.dkcache]
        arrs = []
        for name in ("kcache", "vcache", "dkcache", "dvcache"):
            lst = getattr(self, name)
            arr = (ctypes.c_void_p * max(len(lst), 1))(*[c.ctypes.data for c in lst])
            arrs.append(arr)
            setattr(self.m, name, ctypes.cast(arr, ctypes.c_void_p))
        self._cache_arrs = arrs
        self.cache_B = B


def body_layer(om: OracleModel, l: int, h_in):
    """Body layer l of the frame (identity attention stub) on h_in [B, H]
    (bf16 bits): the residual stream after it, as the oracle frame computes it."""
    cfg = om.cfg
    h = _c(h_in, np.uint16).copy()
    layers = ctypes.cast(om.m.layers, ctypes.POINTER(Layer))
    lib().m3o_layer_stub(ctypes.byref(layers[l]), _ptr(h), h.shape[0], cfg["H"], cfg["n_heads"],
                         cfg["n_kv_heads"], cfg["head_dim"], cfg["F"], float(cfg["eps"]))
    return h


def depth_layer(om: OracleModel, l: int, hd_in):
    """Depth-decoder layer l (identity attention stub) on hd_in [B, D]."""
    cfg = om.cfg
    h = _c(hd_in, np.uint16).copy()
    layers = ctypes.cast(om.m.d_layers_w, ctypes.POINTER(Layer))
    lib().m3o_layer_stub(ctypes.byref(layers[l]), _ptr(h), h.shape[0], cfg["D"], cfg["d_heads"],
                         cfg["d_heads"], cfg["d_head_dim"], cfg["Fd"], float(cfg["eps"]))
    return h


def body_layer_attn(om: OracleModel, l: int, h_in, k_cache, v_cache, pos: int):
    """Body layer l with decode attention at position pos: k_cache, v_cache
    ([B, n_kv, max_pos, 128] bf16 bits) get slot pos written in place; returns
    the residual stream after the layer."""
    cfg = om.cfg
    h = _c(h_in, np.uint16).copy()
    layers = ctypes.cast(om.m.layers, ctypes.POINTER(Layer))
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    lib().m3o_layer_attn(ctypes.byref(layers[l]), _ptr(h), h.shape[0], cfg["H"], cfg["n_heads"],
                         cfg["n_kv_heads"], cfg["head_dim"], cfg["F"], float(cfg["eps"]),
                         om.m.rope, _ptr(k_cache), _ptr(v_cache), k_cache.shape[2], int(pos))
    return h


def depth_layer_attn(om: OracleModel, l: int, hd_in, k_cache, v_cache, pos: int):
    """Depth layer l with attention at codebook position pos over caches
    [B, d_heads, 8, 128] (slot pos written in place)."""
    cfg = om.cfg
    h = _c(hd_in, np.uint16).copy()
    layers = ctypes.cast(om.m.d_layers_w, ctypes.POINTER(Layer))
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    lib().m3o_layer_attn(ctypes.byref(layers[l]), _ptr(h), h.shape[0], cfg["D"], cfg["d_heads"],
                         cfg["d_heads"], cfg["d_head_dim"], cfg["Fd"], float(cfg["eps"]),
                         om.m.rope, _ptr(k_cache), _ptr(v_cache), k_cache.shape[2], int(pos))
    return h


def step_input(om: OracleModel, j: int, codes, u):
    """Depth step j's input bf16(u + Emb_j[c_{j-1}]) from the frame's codes [B, 8]."""
    codes = _c(codes, np.int32)
    u = _c(u, np.uint16)
    out = np.empty_like(u)
    lib().m3o_step_input(ctypes.byref(om.m), int(j), _ptr(codes), _ptr(u), u.shape[0], _ptr(out))
    return out


def feedback(om: OracleModel, codes):
    """The next frame's input bf16((E_tok[c0] + sum_j A_j[c_j]) * 8^-1/2)."""
    codes = _c(codes, np.int32)
    B = codes.shape[0]
    out = np.empty((B, om.cfg["H"]), np.uint16)
    lib().m3o_feedback(ctypes.byref(om.m), _ptr(codes), B, _ptr(out))
    return out


def mat_of(om: OracleModel, which: str, j: int = 0, name: str | None = None) -> Matrix:
    """The oracle's own matrix object, for stage checks: which = "lm_head",
    "p_in" or "head" (depth head j, 1-based); or which = "body" / "depth" with
    layer j and name = "qkv", "o", "gu" (gate/up rows interleaved) or "down"."""
    return om.mats[(which, j) if name is None else (which, j, name)]


def decode_frame(om: OracleModel, x_in, seed, frame, temperature=1.0, trace=False):
    """One frame: returns codes [B, 8] (int32), x_next [B, H] (bf16 bits) and,
    with trace=True, a dict with h_body, logits0 and zgap (decision margins)."""
    x = _c(x_in, np.uint16)
    B, H = x.shape
    cfg = om.cfg
    if om.m.attention and om.cache_B != B:
        om.reset_attention(B)
    codes = np.empty((B, 8), np.int32)
    xn = np.empty((B, H), np.uint16)
    tr_d = None
    tr = FrameTrace(None, None, None)
    if trace:
        tr_d = {"h_body": np.empty((B, H), np.uint16),
                "logits0": np.empty((B, cfg["V0"] + (om.m.end_id >= 0)), np.float32),
                "zgap": np.empty((B, 8), np.float32)}
        tr = FrameTrace(_ptr(tr_d["h_body"]), _ptr(tr_d["logits0"]), _ptr(tr_d["zgap"]))
    lib().m3o_decode_frame(ctypes.byref(om.m), _ptr(x), B, int(seed), int(frame),
                           float(temperature), _ptr(codes), _ptr(xn), ctypes.byref(tr))
    return (codes, xn, tr_d) if trace else (codes, xn)


# ----------------------------------------------------------- weight bytes ---
def matrix_bytes(fmt: int, N: int, K: int) -> int:
    """Algorithmic bytes of one weight matrix: bf16 2NK; int8-row and fp8-row
    NK + 4N; int8-g128 NK + 4N*K/128 (weights plus fp32 scales)."""
    if fmt == BF16:
        return 2 * N * K
    if fmt == I8ROW:
        return N * K + 4 * N
    if fmt == I8G128:
        return N * K + 4 * N * (K // 128)
    if fmt == FP8ROW:
        return N * K + 4 * N
    raise ValueError(fmt)


def frame_weight_bytes(cfg: dict, fmt_body: int, fmt_lm: int, fmt_depth: int) -> int:
    """Weight bytes one frame streams: every body matrix once, the lm_head
    slice once, the depth input projection once, the depth layers once per
    codebook step (7 times) and each step's head once; fp32 norm gammas are
    counted once per norm application (the final body norm once)."""
    H, F = cfg["H"], cfg["F"]
    nq = cfg["n_heads"] * cfg["head_dim"]
    nkv = cfg["n_kv_heads"] * cfg["head_dim"]
    D, Fd = cfg["D"], cfg["Fd"]
    dq = cfg["d_heads"] * cfg["d_head_dim"]
    steps = cfg["n_codebooks"] - 1
    body_layer = (matrix_bytes(fmt_body, nq + 2 * nkv, H) + matrix_bytes(fmt_body, H, nq)
                  + matrix_bytes(fmt_body, 2 * F, H) + matrix_bytes(fmt_body, H, F))
    body = cfg["n_layers"] * body_layer + 4 * H * (2 * cfg["n_layers"] + 1)
    lm = matrix_bytes(fmt_lm, cfg["V0"], H)
    depth_layer = (matrix_bytes(fmt_depth, 3 * dq, D) + matrix_bytes(fmt_depth, D, dq)
                   + matrix_bytes(fmt_depth, 2 * Fd, D) + matrix_bytes(fmt_depth, D, Fd))
    depth_step = (cfg["d_layers"] * depth_layer + matrix_bytes(fmt_depth, cfg["code_vocab"], D)
                  + 4 * D * (2 * cfg["d_layers"] + 1))
    p_in = matrix_bytes(fmt_depth, D, H)
    return body + lm + p_in + steps * depth_step


def num_threads() -> int:
    return int(lib().m3o_num_threads())
