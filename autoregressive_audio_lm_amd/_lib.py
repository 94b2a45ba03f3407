"""ctypes binding of libm3 (argument marshalling only).

Every call goes to the HIP library; there is no fallback.  If libm3.so is
missing the import of the functions raises.  torch tensors supply device
memory and the stream (torch.cuda.current_stream()).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libm3.so")

M3_OK, M3_ERR_NULL, M3_ERR_SHAPE, M3_ERR_ALIGN = 0, -1, -2, -3
M3_ERR_FORMAT, M3_ERR_WORKSPACE, M3_ERR_HIP, M3_ERR_ALIAS = -4, -5, -6, -7
BF16, I8ROW, I8G128, FP8ROW = 0, 1, 2, 3
EPI_NONE, EPI_SWIGLU, EPI_RESIDUAL = 0, 1, 2
OUT_BF16, OUT_F32 = 0, 1
PACK_GLU_INTERLEAVE = 1
MAX_B, MAX_B_FRAME = 64, 16
NOALLOC_SCRATCH_BYTES = 1 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int


class M3Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class M3ValueError(M3Error, ValueError):
    pass


class SampleParams(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("frame", ctypes.c_uint32), ("frame_dev", _P),
                ("draw", ctypes.c_uint32), ("temperature", ctypes.c_float),
                ("index_base", ctypes.c_int32), ("ids", _P), ("valid_lo", ctypes.c_int32),
                ("valid_hi", ctypes.c_int32), ("noise_override", _P)]


class Config(ctypes.Structure):
    _fields_ = [(n, _I) for n in ("hidden", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn",
                                  "vocab_base", "n_slice", "d_hidden", "d_layers", "d_heads",
                                  "d_head_dim", "d_ffn", "n_codebooks", "code_vocab", "fmt_body",
                                  "fmt_lm", "fmt_depth")] + \
               [("eps", ctypes.c_float), ("temperature", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("cfg_scale", ctypes.c_float), ("top_k", _I),
                ("attention", _I), ("max_pos", _I), ("pos0", _I), ("end_id", _I)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("qkv", _P), ("o", _P), ("gate_up", _P), ("down", _P),
                ("attn_norm", _P), ("ffn_norm", _P), ("q_norm", _P), ("k_norm", _P)]


class Model(ctypes.Structure):
    _fields_ = [("cfg", Config), ("layers", _P), ("final_norm", _P), ("lm_head", _P),
                ("p_in", _P), ("emb1", _P), ("emb", _P), ("d_layers_w", _P),
                ("d_final_norm", _P), ("heads", _P), ("tok_emb_audio", _P), ("audio_emb", _P)]


class FrameLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("x", "h", "qkv", "mlp", "logits", "u", "hd", "dqkv",
                                               "dmlp", "dlogits", "ring", "frame", "part_sem", "part_dep",
                                               "flags", "err", "seq", "phases", "th", "tqkv", "tmlp", "tu",
                                               "thd", "tdqkv", "tdmlp", "th2", "thd2", "ho", "hdo", "rope", "aq", "ao", "dao", "kcache",
                                               "vcache", "dkcache", "dvcache", "attn_ws", "tao", "tdao", "trec", "stop",
                                               "kpart", "kcnt", "total")]


class PhaseRegion(ctypes.Structure):
    _fields_ = [("base", ctypes.c_uint64), ("stride", ctypes.c_uint64), ("rows", _I),
                ("c0", ctypes.c_uint32), ("c1", ctypes.c_uint32), ("producer", _I), ("tagged", _I),
                ("pad", _I)]


PHASE_MAX_REGIONS = 4
PHASE_GEMV, PHASE_FRAME_END, PHASE_ATTENTION, PHASE_DRAW = 0, 1, 2, 3


class PhaseRecord(ctypes.Structure):
    _fields_ = [("kind", _I), ("n_in", _I), ("n_out", _I), ("pad", _I),
                ("inp", PhaseRegion * PHASE_MAX_REGIONS), ("out", PhaseRegion * PHASE_MAX_REGIONS)]


M3_ERR_ATTN_FULL = 2      # frame state err word: the frame position reached max_pos

_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "m3_status_str": (ctypes.c_char_p, [_I]),
    "m3_version": (ctypes.c_char_p, []),
    "m3_packed_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "m3_pack": (_I, [_I, _P, _I, _I, _I, _P, _P]),
    "m3_rmsnorm_gemv": (_I, [_P, _I, _I, _P, _I, _I, _P, ctypes.c_float, _I, _I, _P, _I, _I, _I, _P, _I, _P]),
    "m3_gemv_i8row": (_I, [_P, _I, _I, _P, _I, _I, _P, ctypes.c_float, _I, _I, _P, _I, _I, _I, _P, _I, _P]),
    "m3_gemv_i8g128": (_I, [_P, _I, _I, _P, _I, _I, _P, ctypes.c_float, _I, _I, _P, _I, _I, _I, _P, _I, _P]),
    "m3_gemv_fp8row": (_I, [_P, _I, _I, _P, _I, _I, _P, ctypes.c_float, _I, _I, _P, _I, _I, _I, _P, _I, _P]),
    "m3_rmsnorm_rows": (_I, [_P, _I, _I, _I, _P, ctypes.c_float, _P, _I, _P]),
    "m3_prefill_gemm": (_I, [_P, _I, _I, _P, _I, _I, _P, _I, _I, _I, _P, _I, _P]),
    "m3_rope_table": (_I, [_P, _I, _I, ctypes.c_float, _P]),
    "m3_qk_norm_rope": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _I, _P, _I, _P, _P,
                             _I, _P]),
    "m3_attention_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "m3_prefill_qk_norm_rope": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _I, _P,
                                     _I, _P, _P, _I, _P]),
    "m3_prefill_attention_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "m3_prefill_attention": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _I, _P, _I, _P,
                                  ctypes.c_size_t, _P]),
    "m3_decode_attention": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _P, _I, _P, ctypes.c_size_t,
                                 _P]),
    "m3_decode_attention_step": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _I, _P, _P,
                                      _I, _P, _I, _P, ctypes.c_size_t, _P]),
    "m3_lmhead_sliced": (_I, [_I, _P, _I, _I, _P, _I, _I, _P, ctypes.c_float, _P, _I, _P]),
    "m3_gumbel_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "m3_gumbel_argmax": (_I, [_P, _I, _I, _I, ctypes.POINTER(SampleParams), _P, _P, ctypes.c_size_t, _P]),
    "m3_gumbel_argmax_noalloc": (_I, [_P, _I, _I, _I, ctypes.POINTER(SampleParams), _P, _P]),
    "m3_cfg_topk_draw": (_I, [_P, _I, _I, _I, ctypes.c_float, _I, ctypes.POINTER(SampleParams), _P, _P]),
    "m3_frame_weight_bytes": (ctypes.c_uint64, [ctypes.POINTER(Config)]),
    "m3_frame_layout_get": (_I, [ctypes.POINTER(Config), _I, ctypes.POINTER(FrameLayout)]),
    "m3_frame_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config), _I]),
    "m3_frame_state_init": (_I, [ctypes.POINTER(Config), _I, _P, _P, ctypes.c_uint32, _P]),
    "m3_decode_frame_weights": (_I, [ctypes.POINTER(Model), _P, _I, _P, ctypes.POINTER(ctypes.c_uint64), _P]),
    "m3_frame_graph_create": (_I, [ctypes.POINTER(Model), _P, _I, _P, _P, ctypes.POINTER(_P)]),
    "m3_depth_graph_create": (_I, [ctypes.POINTER(Model), _P, _I, _P, _P, ctypes.POINTER(_P)]),
    "m3_frame_graph_launch": (_I, [_P, _P]),
    "m3_frame_graph_destroy": (_I, [_P]),
    "m3_frame_persistent_create": (_I, [ctypes.POINTER(Model), _P, _I, _P, _P, ctypes.POINTER(_P)]),
    "m3_frame_persistent_launch": (_I, [_P, _P]),
    "m3_frame_persistent_destroy": (_I, [_P]),
    "m3_frame_persistent_clock_bytes": (ctypes.c_size_t, [_P]),
    "m3_stream_read": (_I, [_P, ctypes.c_size_t, _P, _I, _I, _P]),
    "m3_frame_phase_table": (_I, [ctypes.POINTER(Model), _P, _I, _P, ctypes.POINTER(PhaseRecord), _I]),
    "m3_frame_persistent_clock": (_I, [_P, _P, ctypes.c_size_t, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
}

SYMBOLS = tuple(_SIGS)


def lib():
    """Load libm3.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libm3.so not built at {LIB_PATH}: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status == M3_OK:
        return
    msg = lib().m3_status_str(status).decode()
    if status == M3_ERR_HIP:
        raise M3Error(status, msg)
    raise M3ValueError(status, msg)


def status_str(status: int) -> str:
    return lib().m3_status_str(status).decode()
