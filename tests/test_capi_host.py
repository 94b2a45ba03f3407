"""Host-side checks of libm3 (no GPU needed): the library loads, exports every
entry point include/m3.h declares, computes sizes, and refuses unsupported
arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

from autoregressive_audio_lm_amd import _lib, configs
from autoregressive_audio_lm_amd.runtime import make_config, frame_weight_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from autoregressive_audio_lm_amd import build
        build.build()
    return _lib.lib()


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "m3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) >= 18
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(_lib.SYMBOLS)


def test_status_strings(L):
    for st in range(0, -8, -1):
        assert L.m3_status_str(st)
    assert b"gfx950" in L.m3_version()


FAKE = ctypes.c_void_p(0x100000)      # aligned, never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x900000)


def gemv(L, fmt=0, N=64, K=256, x=FAKE, B=1, ldx=256, gamma=None, eps=1e-6, sg=0, sv=0, y=FAKE2,
         ldy=64, out=0, epi=0, res=None, ldr=0):
    f = {0: L.m3_rmsnorm_gemv, 1: L.m3_gemv_i8row, 2: L.m3_gemv_i8g128, 3: L.m3_gemv_fp8row}[fmt]
    return f(FAKE, N, K, x, B, ldx, gamma, eps, sg, sv, y, ldy, out, epi, res, ldr, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.M3_ERR_NULL),
    (dict(y=None), _lib.M3_ERR_NULL),
    (dict(B=0), _lib.M3_ERR_SHAPE),
    (dict(B=65), _lib.M3_ERR_SHAPE),
    (dict(N=0), _lib.M3_ERR_SHAPE),
    (dict(K=4, ldx=8), _lib.M3_ERR_SHAPE),
    (dict(K=250), _lib.M3_ERR_SHAPE),
    (dict(fmt=1, K=248, ldx=248), _lib.M3_ERR_SHAPE),       # i8row needs K % 16
    (dict(fmt=3, K=248, ldx=248), _lib.M3_ERR_SHAPE),       # fp8row needs K % 16
    (dict(fmt=2, K=192, ldx=192), _lib.M3_ERR_SHAPE),       # g128 needs K % 128
    (dict(ldx=128), _lib.M3_ERR_SHAPE),
    (dict(ldy=32), _lib.M3_ERR_SHAPE),
    (dict(ldx=260), _lib.M3_ERR_ALIGN),
    (dict(x=ctypes.c_void_p(0x100008)), _lib.M3_ERR_ALIGN),
    (dict(out=7), _lib.M3_ERR_FORMAT),
    (dict(epi=5), _lib.M3_ERR_FORMAT),
    (dict(epi=1, out=1), _lib.M3_ERR_FORMAT),               # SwiGLU writes bf16 only
    (dict(epi=2, res=None), _lib.M3_ERR_NULL),
    (dict(N=63, epi=1), _lib.M3_ERR_SHAPE),                 # SwiGLU needs pairs
    (dict(eps=-1.0), _lib.M3_ERR_SHAPE),
    (dict(eps=float("nan")), _lib.M3_ERR_SHAPE),
    (dict(sg=-1), _lib.M3_ERR_SHAPE),
    (dict(sg=4, sv=0, K=256, ldx=128), _lib.M3_ERR_SHAPE),  # stub: K/128 heads not divisible by 4
    (dict(sg=2, sv=4, K=256, ldx=256), _lib.M3_ERR_SHAPE),  # stub: voff % 8
    (dict(y=ctypes.c_void_p(0x100000 + 64)), _lib.M3_ERR_ALIAS),
    (dict(gamma=FAKE2, K=4096, ldx=4096, B=17, y=ctypes.c_void_p(0x4000000)), _lib.M3_ERR_SHAPE),
])
def test_gemv_refusals(L, kw, status):
    assert gemv(L, **kw) == status


def test_pack_and_sizes(L):
    assert L.m3_packed_bytes(0, 16, 32, 0) == 1024
    assert L.m3_packed_bytes(0, 17, 40, 0) == 2 * 2 * 1024          # 2 blocks x 2 tiles
    assert L.m3_packed_bytes(1, 16, 64, 0) == 1024 + 128            # tile + scales
    assert L.m3_packed_bytes(2, 16, 256, 0) == 4 * 1024 + 128       # 2 groups x 64 B -> 128
    assert L.m3_packed_bytes(2, 16, 200, 0) == 0
    assert L.m3_packed_bytes(0, 15, 64, 1) == 0                     # GLU needs even N
    assert L.m3_packed_bytes(3, 16, 64, 0) == 1024 + 128            # fp8-row: as int8-row
    assert L.m3_packed_bytes(4, 16, 64, 0) == 0                     # unknown format
    assert L.m3_pack(0, None, 16, 32, 0, FAKE, None) == _lib.M3_ERR_NULL
    assert L.m3_pack(0, FAKE, 16, 30, 0, FAKE2, None) == _lib.M3_ERR_SHAPE
    assert L.m3_pack(5, FAKE, 16, 32, 0, FAKE2, None) == _lib.M3_ERR_FORMAT


def test_sampler_refusals(L):
    p = _lib.SampleParams(0, 0, None, 0, 1.0, 0, None, 0, 0, None)
    ws = L.m3_gumbel_workspace_bytes(4, 5000)
    assert ws == 4 * 5 * 8
    arg = lambda **k: (k.get("lg", FAKE), k.get("B", 4), k.get("V", 5000), k.get("ldl", 5000),
                       ctypes.byref(k.get("p", p)), k.get("out", FAKE2), k.get("ws", ctypes.c_void_p(0x2000000)),
                       k.get("wsb", ws), None)
    assert L.m3_gumbel_argmax(*arg(lg=None)) == _lib.M3_ERR_NULL
    assert L.m3_gumbel_argmax(*arg(B=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_gumbel_argmax(*arg(ldl=4000)) == _lib.M3_ERR_SHAPE
    assert L.m3_gumbel_argmax(*arg(wsb=ws - 1)) == _lib.M3_ERR_WORKSPACE
    assert L.m3_gumbel_argmax(*arg(lg=ctypes.c_void_p(0x100002))) == _lib.M3_ERR_ALIGN
    assert L.m3_gumbel_argmax(*arg(B=65536)) == _lib.M3_ERR_SHAPE
    bad = _lib.SampleParams(0, 0, None, 0, 0.0, 0, None, 0, 0, None)
    assert L.m3_gumbel_argmax(*arg(p=bad)) == _lib.M3_ERR_SHAPE


def test_noalloc_sampler_refusals(L):
    """The allocation-free draw checks every argument, and refuses a draw
    whose winners do not fit the library's fixed scratch, before it looks up
    the scratch or launches anything."""
    p = _lib.SampleParams(0, 0, None, 0, 1.0, 0, None, 0, 0, None)
    f = L.m3_gumbel_argmax_noalloc
    assert f(None, 4, 5000, 5000, ctypes.byref(p), FAKE2, None) == _lib.M3_ERR_NULL
    assert f(FAKE, 4, 5000, 5000, None, FAKE2, None) == _lib.M3_ERR_NULL
    assert f(FAKE, 0, 5000, 5000, ctypes.byref(p), FAKE2, None) == _lib.M3_ERR_SHAPE
    assert f(FAKE, 4, 5000, 4000, ctypes.byref(p), FAKE2, None) == _lib.M3_ERR_SHAPE
    assert f(ctypes.c_void_p(0x100002), 4, 5000, 5000, ctypes.byref(p), FAKE2, None) == _lib.M3_ERR_ALIGN
    bad = _lib.SampleParams(0, 0, None, 0, 0.0, 0, None, 0, 0, None)
    assert f(FAKE, 4, 5000, 5000, ctypes.byref(bad), FAKE2, None) == _lib.M3_ERR_SHAPE
    # 16 rows of 2^24 columns: 16 * 16384 chunk winners of 8 bytes = 2 MiB > 1 MiB
    assert L.m3_gumbel_workspace_bytes(16, 1 << 24) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, 16, 1 << 24, 1 << 24, ctypes.byref(p), FAKE2, None) == _lib.M3_ERR_WORKSPACE
    assert L.m3_gumbel_workspace_bytes(8, 1 << 24) == _lib.NOALLOC_SCRATCH_BYTES


def test_stream_read_and_depth_graph_refusals(L):
    """The streaming-read measurement and the depth decoder's graph check
    their arguments before anything is launched or captured."""
    f = L.m3_stream_read
    assert f(None, 1 << 20, FAKE2, 256, 1, None) == _lib.M3_ERR_NULL
    assert f(FAKE, 1 << 20, None, 256, 1, None) == _lib.M3_ERR_NULL
    assert f(FAKE, 0, FAKE2, 256, 1, None) == _lib.M3_ERR_SHAPE
    assert f(FAKE, (1 << 20) + 8, FAKE2, 256, 1, None) == _lib.M3_ERR_SHAPE
    assert f(FAKE, 1 << 31, FAKE2, 256, 1, None) == _lib.M3_ERR_SHAPE
    assert f(FAKE, 1 << 20, FAKE2, 0, 1, None) == _lib.M3_ERR_SHAPE
    assert f(FAKE, 1 << 20, FAKE2, 4097, 1, None) == _lib.M3_ERR_SHAPE
    assert f(ctypes.c_void_p(0x100008), 1 << 20, FAKE2, 256, 1, None) == _lib.M3_ERR_ALIGN
    g = ctypes.c_void_p()
    assert L.m3_depth_graph_create(None, FAKE, 1, FAKE2, FAKE, ctypes.byref(g)) == _lib.M3_ERR_NULL


def test_prefill_refusals(L):
    arg = lambda **k: (k.get("w", FAKE), k.get("N", 256), k.get("K", 512), k.get("a", FAKE2),
                       k.get("M", 600), k.get("lda", 512), k.get("y", ctypes.c_void_p(0x4000000)),
                       k.get("ldy", 256), k.get("out", 0), k.get("epi", 0), k.get("res", None),
                       k.get("ldr", 0), None)
    assert L.m3_prefill_gemm(*arg(w=None)) == _lib.M3_ERR_NULL
    assert L.m3_prefill_gemm(*arg(M=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_prefill_gemm(*arg(K=480, lda=480)) == _lib.M3_ERR_SHAPE     # K % 64
    assert L.m3_prefill_gemm(*arg(lda=256)) == _lib.M3_ERR_SHAPE
    assert L.m3_prefill_gemm(*arg(ldy=128)) == _lib.M3_ERR_SHAPE
    assert L.m3_prefill_gemm(*arg(epi=1, N=255)) == _lib.M3_ERR_SHAPE      # SwiGLU pairs
    assert L.m3_prefill_gemm(*arg(epi=2)) == _lib.M3_ERR_NULL               # residual missing
    assert L.m3_prefill_gemm(*arg(epi=1, out=1)) == _lib.M3_ERR_FORMAT
    assert L.m3_prefill_gemm(*arg(out=7)) == _lib.M3_ERR_FORMAT
    assert L.m3_prefill_gemm(*arg(a=ctypes.c_void_p(0x900008))) == _lib.M3_ERR_ALIGN
    assert L.m3_prefill_gemm(*arg(y=FAKE2)) == _lib.M3_ERR_ALIAS
    g = ctypes.c_void_p(0x5000000)
    assert L.m3_rmsnorm_rows(None, 4, 64, 64, g, 1e-6, FAKE2, 64, None) == _lib.M3_ERR_NULL
    assert L.m3_rmsnorm_rows(FAKE, 4, 60, 64, g, 1e-6, FAKE2, 64, None) == _lib.M3_ERR_SHAPE
    assert L.m3_rmsnorm_rows(FAKE, 4, 64, 64, g, -1.0, FAKE2, 64, None) == _lib.M3_ERR_SHAPE
    assert L.m3_rmsnorm_rows(FAKE, 4, 64, 64, g, 1e-6, FAKE, 64, None) == _lib.M3_ERR_ALIAS


def test_attention_refusals(L):
    """Decode attention: sizes, head groups, alignment, workspace and aliasing
    are refused on the host, before any launch."""
    P = ctypes.c_void_p

    assert L.m3_attention_workspace_bytes(1, 32, 8, 64) == 0                    # one chunk of 64
    assert L.m3_attention_workspace_bytes(1, 32, 8, 65) == 32 * 2 * 130 * 4
    assert L.m3_attention_workspace_bytes(1, 32, 8, 1800) == 32 * 29 * 130 * 4   # 64 wide
    assert L.m3_attention_workspace_bytes(16, 32, 8, 1800) == 16 * 32 * 15 * 130 * 4
    assert L.m3_attention_workspace_bytes(2, 32, 8, 128) == 2 * 32 * 2 * 130 * 4
    assert L.m3_attention_workspace_bytes(2, 24, 8, 300) == 0                   # unsupported heads
    tab = P(0x1000000)
    assert L.m3_rope_table(None, 16, 128, 1e6, None) == _lib.M3_ERR_NULL
    assert L.m3_rope_table(tab, 16, 64, 1e6, None) == _lib.M3_ERR_SHAPE
    assert L.m3_rope_table(tab, 0, 128, 1e6, None) == _lib.M3_ERR_SHAPE
    assert L.m3_rope_table(tab, 16, 128, 0.5, None) == _lib.M3_ERR_SHAPE
    assert L.m3_rope_table(P(0x1000004), 16, 128, 1e6, None) == _lib.M3_ERR_ALIGN
    # qk norm + rope: B = 2, 32 q heads over 8 KV heads, caches of 64 positions
    cb = 2 * 8 * 64 * 128 * 2
    q_arg = lambda **k: (k.get("qkv", P(0x10000000)), k.get("B", 2), k.get("ldqkv", 6144),
                         k.get("nq", 32), k.get("nkv", 8), k.get("hd", 128), k.get("qg", P(0x30000000)),
                         k.get("kg", P(0x30001000)), k.get("eps", 1e-6), k.get("rope", tab),
                         k.get("pos", 5), k.get("qo", P(0x20000000)), k.get("ldq", 4096),
                         k.get("kc", P(0x40000000)), k.get("vc", P(0x40000000 + cb)),
                         k.get("mp", 64), None)
    assert L.m3_qk_norm_rope(*q_arg(qkv=None)) == _lib.M3_ERR_NULL
    assert L.m3_qk_norm_rope(*q_arg(hd=64)) == _lib.M3_ERR_SHAPE
    assert L.m3_qk_norm_rope(*q_arg(nq=24)) == _lib.M3_ERR_SHAPE        # 3 q heads per KV head
    assert L.m3_qk_norm_rope(*q_arg(nq=4, nkv=8)) == _lib.M3_ERR_SHAPE
    assert L.m3_qk_norm_rope(*q_arg(pos=64)) == _lib.M3_ERR_SHAPE
    assert L.m3_qk_norm_rope(*q_arg(ldqkv=6000)) == _lib.M3_ERR_SHAPE
    assert L.m3_qk_norm_rope(*q_arg(B=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_qk_norm_rope(*q_arg(qo=P(0x20000008))) == _lib.M3_ERR_ALIGN
    assert L.m3_qk_norm_rope(*q_arg(vc=P(0x40000000 + cb - 256))) == _lib.M3_ERR_ALIAS
    assert L.m3_qk_norm_rope(*q_arg(qo=P(0x10000000 + 4096))) == _lib.M3_ERR_ALIAS
    # attention: T = 300 needs workspace (five chunks of 64 at B * n_kv = 16)
    need = L.m3_attention_workspace_bytes(2, 32, 8, 300)
    a_arg = lambda **k: (k.get("q", P(0x20000000)), k.get("B", 2), k.get("ldq", 4096), k.get("nq", 32),
                         k.get("nkv", 8), k.get("hd", 128), k.get("kc", P(0x40000000)),
                         k.get("vc", P(0x48000000)), k.get("mp", 512), k.get("T", 300),
                         k.get("out", P(0x50000000)), k.get("ldo", 4096), k.get("ws", P(0x60000000)),
                         k.get("wsb", need), None)
    assert L.m3_decode_attention(*a_arg(out=None)) == _lib.M3_ERR_NULL
    assert L.m3_decode_attention(*a_arg(ws=None)) == _lib.M3_ERR_NULL
    assert L.m3_decode_attention(*a_arg(wsb=need - 1)) == _lib.M3_ERR_WORKSPACE
    assert L.m3_decode_attention(*a_arg(T=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention(*a_arg(T=513)) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention(*a_arg(nq=48, nkv=3)) == _lib.M3_ERR_SHAPE   # 16 per KV head
    assert L.m3_decode_attention(*a_arg(ldo=4000)) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention(*a_arg(out=P(0x50000002))) == _lib.M3_ERR_ALIGN
    assert L.m3_decode_attention(*a_arg(out=P(0x20000000 + 64))) == _lib.M3_ERR_ALIAS
    assert L.m3_decode_attention(*a_arg(ws=P(0x40000000))) == _lib.M3_ERR_ALIAS
    # one chunk: no workspace needed
    assert L.m3_attention_workspace_bytes(2, 16, 16, 64) == 0
    # the one-launch step: qk norm + rope at pos, attention over pos + 1 positions
    need_s = L.m3_attention_workspace_bytes(2, 32, 8, 300)
    s_arg = lambda **k: (k.get("qkv", P(0x10000000)), k.get("B", 2), k.get("ldqkv", 6144),
                         k.get("nq", 32), k.get("nkv", 8), k.get("hd", 128), P(0x30000000),
                         P(0x30001000), k.get("eps", 1e-6), tab, k.get("pos", 299),
                         k.get("kc", P(0x40000000)), k.get("vc", P(0x48000000)), k.get("mp", 512),
                         k.get("out", P(0x50000000)), k.get("ldo", 4096), k.get("ws", P(0x60000000)),
                         k.get("wsb", need_s), None)
    assert L.m3_decode_attention_step(*s_arg(qkv=None)) == _lib.M3_ERR_NULL
    assert L.m3_decode_attention_step(*s_arg(ws=None)) == _lib.M3_ERR_NULL
    assert L.m3_decode_attention_step(*s_arg(wsb=need_s - 1)) == _lib.M3_ERR_WORKSPACE
    assert L.m3_decode_attention_step(*s_arg(pos=512)) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention_step(*s_arg(nq=24)) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention_step(*s_arg(eps=float("nan"))) == _lib.M3_ERR_SHAPE
    assert L.m3_decode_attention_step(*s_arg(out=P(0x50000002))) == _lib.M3_ERR_ALIGN
    assert L.m3_decode_attention_step(*s_arg(vc=P(0x40000000 + 4096))) == _lib.M3_ERR_ALIAS
    assert L.m3_decode_attention_step(*s_arg(out=P(0x10000000 + 4096))) == _lib.M3_ERR_ALIAS
    assert L.m3_decode_attention_step(*s_arg(ws=P(0x48000000))) == _lib.M3_ERR_ALIAS


def test_prompt_attention_refusals(L):
    P = ctypes.c_void_p
    need = L.m3_prefill_attention_workspace_bytes(2, 300, 32, 8, 0)
    assert need == 0                                     # the tiled kernel keeps no records
    tab = P(0x1000000)
    cb = 2 * 8 * 512 * 128 * 2
    q_arg = lambda **k: (k.get("qkv", P(0x10000000)), k.get("S", 2), k.get("L", 300),
                         k.get("ld", 6144), 32, 8, 128, P(0x30000000), P(0x30001000), 1e-6, tab,
                         k.get("pb", 0), k.get("qo", P(0x20000000)), 4096, P(0x40000000),
                         P(0x40000000 + cb), k.get("mp", 512), None)
    assert L.m3_prefill_qk_norm_rope(*q_arg(qkv=None)) == _lib.M3_ERR_NULL
    assert L.m3_prefill_qk_norm_rope(*q_arg(pb=300)) == _lib.M3_ERR_SHAPE    # past max_pos
    assert L.m3_prefill_qk_norm_rope(*q_arg(S=65)) == _lib.M3_ERR_SHAPE
    assert L.m3_prefill_qk_norm_rope(*q_arg(ld=6000)) == _lib.M3_ERR_SHAPE
    assert L.m3_prefill_qk_norm_rope(*q_arg(qo=P(0x20000004))) == _lib.M3_ERR_ALIGN
    assert L.m3_prefill_qk_norm_rope(*q_arg(qo=P(0x10000000 + 8192))) == _lib.M3_ERR_ALIAS
    a_arg = lambda **k: (P(0x20000000), k.get("S", 2), k.get("L", 300), 4096, 32, k.get("nkv", 8), 128,
                         P(0x40000000), P(0x40000000 + cb), k.get("mp", 512), k.get("pb", 0),
                         k.get("out", P(0x50000000)), 4096, k.get("ws", P(0x60000000)),
                         k.get("wsb", need), None)
    assert L.m3_prefill_attention(*a_arg(out=None)) == _lib.M3_ERR_NULL
    assert L.m3_prefill_attention(*a_arg(nkv=7)) == _lib.M3_ERR_SHAPE        # 32 heads over 7
    assert L.m3_prefill_attention(*a_arg(pb=213)) == _lib.M3_ERR_SHAPE        # 213 + 300 > 512
    assert L.m3_prefill_attention(*a_arg(out=P(0x20000000 + 64))) == _lib.M3_ERR_ALIAS


def test_cfg_draw_refusals(L):
    p = _lib.SampleParams(0, 0, None, 0, 1.0, 0, None, 0, 0, None)
    arg = lambda **k: (k.get("lg", FAKE), k.get("S", 4), k.get("V", 5000), k.get("ldl", 5000),
                       k.get("scale", 1.5), k.get("k", 50), ctypes.byref(k.get("p", p)),
                       k.get("out", FAKE2), None)
    assert L.m3_cfg_topk_draw(*arg(lg=None)) == _lib.M3_ERR_NULL
    assert L.m3_cfg_topk_draw(*arg(out=None)) == _lib.M3_ERR_NULL
    assert L.m3_cfg_topk_draw(*arg(S=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(S=32768)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(V=0, ldl=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(V=32769, ldl=32769)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(ldl=4999)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(k=0)) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(scale=float("inf"))) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(scale=float("nan"))) == _lib.M3_ERR_SHAPE
    assert L.m3_cfg_topk_draw(*arg(lg=ctypes.c_void_p(0x100002))) == _lib.M3_ERR_ALIGN
    bad = _lib.SampleParams(0, 0, None, 0, -1.0, 0, None, 0, 0, None)
    assert L.m3_cfg_topk_draw(*arg(p=bad)) == _lib.M3_ERR_SHAPE


@pytest.mark.parametrize("preset", ["A", "B", "C"])
@pytest.mark.parametrize("name", ["frame-full", "frame-small"])
def test_frame_weight_bytes_matches_oracle_formula(L, oracle, preset, name):
    cfg = configs.config(name)
    p = configs.PRESETS[preset]
    c = make_config(cfg, **p)
    assert frame_weight_bytes(c) == oracle.frame_weight_bytes(cfg, **p)


def test_frame_layout_and_refusals(L):
    cfg = configs.config("frame-full")
    c = make_config(cfg, **configs.PRESETS["A"])
    lay = _lib.FrameLayout()
    assert L.m3_frame_layout_get(ctypes.byref(c), 16, ctypes.byref(lay)) == 0
    assert lay.total % 256 == 0 and lay.x == 0 and lay.total > lay.part_dep > lay.part_sem > lay.frame
    # the persistent frame's streams: tagged 32-bit words, O's outputs in their own regions
    names = ("th", "tqkv", "tmlp", "tu", "thd", "tdqkv", "tdmlp", "th2", "thd2", "rope")
    offs = [getattr(lay, n) for n in names]
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    assert lay.thd2 - lay.th2 >= 16 * cfg["H"] * 4 and lay.rope - lay.thd2 >= 16 * cfg["D"] * 4
    assert lay.tqkv - lay.th >= 16 * cfg["H"] * 4 and lay.tdqkv - lay.thd >= 16 * cfg["D"] * 4
    assert L.m3_frame_workspace_bytes(ctypes.byref(c), 17) == 0
    assert L.m3_frame_layout_get(ctypes.byref(c), 0, ctypes.byref(lay)) == _lib.M3_ERR_SHAPE
    c2 = make_config(cfg, 0, 2, 2)                                   # lm_head must be bf16/i8row
    assert L.m3_frame_layout_get(ctypes.byref(c2), 1, ctypes.byref(lay)) == _lib.M3_ERR_FORMAT
    c3 = make_config(dict(cfg, head_dim=64), **configs.PRESETS["A"])
    assert L.m3_frame_layout_get(ctypes.byref(c3), 1, ctypes.byref(lay)) == _lib.M3_ERR_SHAPE
    # the reference's draw: rows come in (conditional, unconditional) pairs
    g = make_config(cfg, **configs.PRESETS["A"], top_k=50)
    assert L.m3_frame_layout_get(ctypes.byref(g), 4, ctypes.byref(lay)) == 0
    assert L.m3_frame_layout_get(ctypes.byref(g), 3, ctypes.byref(lay)) == _lib.M3_ERR_SHAPE
    g_bad = make_config(cfg, **configs.PRESETS["A"], top_k=-1)
    assert L.m3_frame_layout_get(ctypes.byref(g_bad), 2, ctypes.byref(lay)) == _lib.M3_ERR_SHAPE
    g_nan = make_config(cfg, **configs.PRESETS["A"], top_k=50, cfg_scale=float("nan"))
    assert L.m3_frame_layout_get(ctypes.byref(g_nan), 2, ctypes.byref(lay)) == _lib.M3_ERR_SHAPE
    m = _lib.Model(cfg=c)
    codes = ctypes.c_void_p(0x300000)
    assert L.m3_decode_frame_weights(ctypes.byref(m), FAKE, 1, codes, None, None) == _lib.M3_ERR_NULL


@pytest.mark.parametrize("name,B", [("frame-full", 1), ("frame-full", 16), ("frame-small", 3)])
def test_frame_layout_stage_slots(L, name, B):
    """Every GEMV output of every body layer and of every depth layer of every
    codebook step, every depth step's input and every depth head's logits has
    a slot of its own in the state (plain and tagged), so each operation of a
    frame can be checked from the input it was given; the slots are laid out
    in the documented order and sizes."""
    cfg = configs.config(name)
    c = make_config(cfg, **configs.PRESETS["A"])
    lay = _lib.FrameLayout()
    assert L.m3_frame_layout_get(ctypes.byref(c), B, ctypes.byref(lay)) == 0
    nL, S, DL = cfg["n_layers"], cfg["n_codebooks"] - 1, cfg["d_layers"]
    nqkv = (cfg["n_heads"] + 2 * cfg["n_kv_heads"]) * 128
    dqkv = 3 * cfg["d_heads"] * 128
    order = ["x", "h", "qkv", "mlp", "logits", "u", "hd", "dqkv", "dmlp", "dlogits", "ring"]
    need = {"x": B * cfg["H"] * 2, "h": nL * B * cfg["H"] * 2, "qkv": nL * B * nqkv * 2,
            "mlp": nL * B * cfg["F"] * 2, "logits": B * cfg["V0"] * 4, "u": B * cfg["D"] * 2,
            "hd": S * (DL + 1) * B * cfg["D"] * 2, "dqkv": S * DL * B * dqkv * 2,
            "dmlp": S * DL * B * cfg["Fd"] * 2, "dlogits": S * B * cfg["code_vocab"] * 4}
    for a, b in zip(order, order[1:]):
        span = getattr(lay, b) - getattr(lay, a)
        assert need[a] <= span < need[a] + 256, (a, span, need[a])
    tagged = ["th", "tqkv", "tmlp", "tu", "thd", "tdqkv", "tdmlp", "th2", "thd2", "ho", "hdo", "rope"]
    tneed = {"th": 2 * need["h"], "tqkv": 2 * need["qkv"], "tmlp": 2 * need["mlp"], "tu": 2 * need["u"],
             "thd": 2 * need["hd"], "tdqkv": 2 * need["dqkv"], "tdmlp": 2 * need["dmlp"],
             "th2": nL * B * cfg["H"] * 4, "thd2": S * DL * B * cfg["D"] * 4,
             "ho": nL * B * cfg["H"] * 2, "hdo": S * DL * B * cfg["D"] * 2}
    for a, b in zip(tagged, tagged[1:]):
        span = getattr(lay, b) - getattr(lay, a)
        assert tneed[a] <= span < tneed[a] + 256, (a, span, tneed[a])
    # without attention the attention buffers take no room; the rows' stop
    # words come next, then the split-K scratch of the down projections (fp32
    # partials of 8 waves x 16 rows x 16 outputs per row block of
    # max(H, D) rows; a counter per group of 4 row blocks)
    assert lay.rope == lay.aq == lay.ao == lay.dao == lay.kcache == lay.trec == lay.stop
    up = lambda n: (n + 255) // 256 * 256
    nb = (max(cfg["H"], cfg["D"]) + 15) // 16
    assert lay.kpart == lay.stop + up(B * 4)
    assert lay.kcnt == lay.kpart + up(nb * 8 * 16 * 16 * 4)
    assert lay.total == lay.kcnt + up((nb + 3) // 4 * 4)
    # with the end token the semantic logits have one more column (rows padded to 8)
    ce = make_config(cfg, **configs.PRESETS["A"], end_token=True)
    le = _lib.FrameLayout()
    assert L.m3_frame_layout_get(ctypes.byref(ce), B, ctypes.byref(le)) == 0
    ldl = (cfg["V0"] + 1 + 7) // 8 * 8
    assert B * ldl * 4 <= le.u - le.logits < B * ldl * 4 + 256
    bad = make_config(cfg, **configs.PRESETS["A"])
    bad.end_id = cfg["vocab_base"]                  # the end token sorts before the codes
    assert L.m3_frame_layout_get(ctypes.byref(bad), B, ctypes.byref(le)) == _lib.M3_ERR_SHAPE


def test_frame_layout_with_attention(L):
    """attention = 1 adds the RoPE table, q/out buffers, the body and depth
    caches and the attention workspace to the state (zero-sized otherwise);
    the sizes follow the documented layouts."""
    cfg = configs.config("frame-full")
    B, max_pos = 2, 2048
    plain = make_config(cfg, **configs.PRESETS["A"])
    att = make_config(cfg, **configs.PRESETS["A"], attention=1, max_pos=max_pos, pos0=300)
    lp, la = _lib.FrameLayout(), _lib.FrameLayout()
    assert L.m3_frame_layout_get(ctypes.byref(plain), B, ctypes.byref(lp)) == 0
    assert L.m3_frame_layout_get(ctypes.byref(att), B, ctypes.byref(la)) == 0
    # the plain layout is unchanged by the attention fields
    assert lp.stop == lp.rope == lp.kcache == lp.attn_ws
    assert la.dao - la.ao >= cfg["n_layers"] * B * cfg["n_heads"] * 128 * 2
    assert la.kcache - la.dao >= (cfg["n_codebooks"] - 1) * cfg["d_layers"] * B * cfg["D"] * 2
    kv = cfg["n_layers"] * B * cfg["n_kv_heads"] * max_pos * 128 * 2
    assert la.vcache - la.kcache >= kv and la.dkcache - la.vcache >= kv
    dkv = cfg["d_layers"] * B * cfg["d_heads"] * 8 * 128 * 2
    assert la.dvcache - la.dkcache >= dkv and la.attn_ws - la.dvcache >= dkv
    assert la.aq - la.rope >= max_pos * 64 * 2 * 4
    assert la.tao - la.attn_ws == L.m3_attention_workspace_bytes(B, cfg["n_heads"],
                                                                  cfg["n_kv_heads"], max_pos)
    # the persistent frame's attention outputs (u32 words) and chunk records:
    # at B = 2 over 2048 positions, chunks of 128 (2 rows x 8 KV heads x 16
    # chunks fill 256 workgroups), 16 chunks of [2 + 128] 64-bit words per
    # row and query head
    assert la.tdao - la.tao == cfg["n_layers"] * B * cfg["n_heads"] * 128 * 4
    assert la.trec - la.tdao == (cfg["n_codebooks"] - 1) * cfg["d_layers"] * B * cfg["D"] * 4
    assert la.stop - la.trec == cfg["n_layers"] * B * cfg["n_heads"] * 16 * 130 * 8
    assert lp.tao == lp.tdao == lp.trec == lp.stop
    assert la.total > lp.total + 2 * kv
    # attention settings out of range are refused
    for bad in (dict(attention=2, max_pos=16), dict(attention=1, max_pos=0),
                dict(attention=1, max_pos=16, pos0=16), dict(attention=1, max_pos=70000),
                dict(attention=1, max_pos=16, pos0=-1)):
        c = make_config(cfg, **configs.PRESETS["A"], **bad)
        assert L.m3_frame_layout_get(ctypes.byref(c), B, ctypes.byref(la)) == _lib.M3_ERR_SHAPE
    # GQA groups other than 1, 2, 4, 8 query heads per KV head are refused
    c = make_config(dict(cfg, n_heads=24), **configs.PRESETS["A"], attention=1, max_pos=16)
    assert L.m3_frame_layout_get(ctypes.byref(c), B, ctypes.byref(la)) == _lib.M3_ERR_SHAPE
