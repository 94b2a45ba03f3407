"""Python binding of the libm3 C ABI, same names as the C entry points.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step runs in libm3's kernels.  Validation refusals
raise ValueError (M3ValueError), HIP failures RuntimeError (M3Error).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (BF16, I8ROW, I8G128, FP8ROW, EPI_NONE, EPI_SWIGLU, EPI_RESIDUAL, OUT_BF16, OUT_F32,
                   PACK_GLU_INTERLEAVE, check, lib)

__all__ = ["packed_bytes", "pack", "rmsnorm_gemv", "gemv_i8row", "gemv_i8g128", "gemv_fp8row", "gemv", "cfg_topk_draw", "rmsnorm_rows", "prefill_gemm",
           "lmhead_sliced", "gumbel_workspace_bytes", "gumbel_argmax", "gumbel_argmax_noalloc", "BF16", "I8ROW", "I8G128", "FP8ROW",
           "EPI_NONE", "EPI_SWIGLU", "EPI_RESIDUAL", "OUT_BF16", "OUT_F32", "PACK_GLU_INTERLEAVE"]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _cuda(t, name):
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def packed_bytes(fmt: int, N: int, K: int, flags: int = 0) -> int:
    return int(lib().m3_packed_bytes(fmt, N, K, flags))


def pack(fmt: int, W: torch.Tensor, flags: int = 0, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """Quantise (int8 formats) and pack a bf16 [N, K] weight on the GPU."""
    _cuda(W, "W")
    if W.dtype != torch.bfloat16 or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous bf16 [N, K] tensor")
    N, K = W.shape
    nb = packed_bytes(fmt, N, K, flags)
    if nb == 0:
        raise ValueError(f"unsupported pack shape fmt={fmt} N={N} K={K} flags={flags}")
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=W.device)
    check(lib().m3_pack(fmt, _ptr(W), N, K, flags, _ptr(out), _stream(stream)))
    return out


_GEMV = {BF16: "m3_rmsnorm_gemv", I8ROW: "m3_gemv_i8row", I8G128: "m3_gemv_i8g128",
         FP8ROW: "m3_gemv_fp8row"}


def gemv(fmt: int, packed: torch.Tensor, N: int, K: int, x: torch.Tensor,
         gamma: torch.Tensor | None = None, eps: float = 1e-6, stub_group: int = 0,
         stub_voff: int = 0, y: torch.Tensor | None = None, out_dtype: int = OUT_BF16,
         epi: int = EPI_NONE, residual: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = epi(W . rmsnorm(x; gamma, eps)) through the C ABI (see m3.h)."""
    for t, n in ((packed, "packed"), (x, "x"), (gamma, "gamma"), (y, "y"), (residual, "residual")):
        _cuda(t, n)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a bf16 [B, ldx] tensor")
    B = x.shape[0]
    ncols = N // 2 if epi == EPI_SWIGLU else N
    if y is None:
        y = torch.empty(B, ncols, dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                        device=x.device)
    ldr = residual.stride(0) if residual is not None else 0
    check(getattr(lib(), _GEMV[fmt])(
        _ptr(packed), N, K, _ptr(x), B, x.stride(0), _ptr(gamma), float(eps), stub_group, stub_voff,
        _ptr(y), y.stride(0), out_dtype, epi, _ptr(residual), ldr, _stream(stream)))
    return y


def rmsnorm_gemv(packed, N, K, x, **kw):
    return gemv(BF16, packed, N, K, x, **kw)


def gemv_i8row(packed, N, K, x, **kw):
    return gemv(I8ROW, packed, N, K, x, **kw)


def gemv_i8g128(packed, N, K, x, **kw):
    return gemv(I8G128, packed, N, K, x, **kw)


def gemv_fp8row(packed, N, K, x, **kw):
    return gemv(FP8ROW, packed, N, K, x, **kw)


def lmhead_sliced(fmt: int, packed: torch.Tensor, n_rows: int, K: int, x: torch.Tensor,
                  gamma: torch.Tensor | None, eps: float = 1e-6,
                  logits: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _cuda(packed, "packed")
    _cuda(x, "x")
    _cuda(gamma, "gamma")
    B = x.shape[0]
    if logits is None:
        logits = torch.empty(B, n_rows, dtype=torch.float32, device=x.device)
    check(lib().m3_lmhead_sliced(fmt, _ptr(packed), n_rows, K, _ptr(x), B, x.stride(0),
                                 _ptr(gamma), float(eps), _ptr(logits), logits.stride(0),
                                 _stream(stream)))
    return logits


def gumbel_workspace_bytes(B: int, V: int) -> int:
    return int(lib().m3_gumbel_workspace_bytes(B, V))


def gumbel_argmax(logits: torch.Tensor, seed: int = 0, frame: int = 0, draw: int = 0,
                  temperature: float = 1.0, index_base: int = 0, ids: torch.Tensor | None = None,
                  valid=(0, 0), noise: torch.Tensor | None = None,
                  frame_dev: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    for t, n in ((logits, "logits"), (ids, "ids"), (noise, "noise"), (frame_dev, "frame_dev"),
                 (out, "out"), (workspace, "workspace")):
        _cuda(t, n)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a float32 [B, V] tensor")
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    need = gumbel_workspace_bytes(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    p = _lib.SampleParams(int(seed) & (2**64 - 1), int(frame), _ptr(frame_dev), int(draw),
                          float(temperature), int(index_base), _ptr(ids), int(valid[0]),
                          int(valid[1]), _ptr(noise))
    check(lib().m3_gumbel_argmax(_ptr(logits), B, V, logits.stride(0), ctypes.byref(p), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def gumbel_argmax_noalloc(logits: torch.Tensor, seed: int = 0, frame: int = 0, draw: int = 0,
                          temperature: float = 1.0, index_base: int = 0,
                          ids: torch.Tensor | None = None, valid=(0, 0),
                          noise: torch.Tensor | None = None, frame_dev: torch.Tensor | None = None,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_gumbel_argmax_noalloc: the same draw with the library's fixed
    per-device scratch in place of a workspace (nothing is allocated when
    `out` is given)."""
    for t, n in ((logits, "logits"), (ids, "ids"), (noise, "noise"), (frame_dev, "frame_dev"),
                 (out, "out")):
        _cuda(t, n)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a float32 [B, V] tensor")
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    p = _lib.SampleParams(int(seed) & (2**64 - 1), int(frame), _ptr(frame_dev), int(draw),
                          float(temperature), int(index_base), _ptr(ids), int(valid[0]),
                          int(valid[1]), _ptr(noise))
    check(lib().m3_gumbel_argmax_noalloc(_ptr(logits), B, V, logits.stride(0), ctypes.byref(p),
                                         _ptr(out), _stream(stream)))
    return out


def stream_read(buf: torch.Tensor, workgroups: int, nontemporal: bool = True,
                sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_stream_read: a plain streaming read of buf (a contiguous device
    tensor) by `workgroups` workgroups; returns the sink words."""
    _cuda(buf, "buf")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    check(lib().m3_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                               int(workgroups), int(bool(nontemporal)), _stream(stream)))
    return sink


def cfg_topk_draw(logits: torch.Tensor, scale: float = 1.5, top_k: int = 50, seed: int = 0,
                  frame: int = 0, draw: int = 0, temperature: float = 1.0, index_base: int = 0,
                  ids: torch.Tensor | None = None, valid=(0, 0),
                  noise: torch.Tensor | None = None, frame_dev: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_cfg_topk_draw: logits float32 [2S, V] (rows 2s conditional, 2s+1
    unconditional) -> int32 [2S], both rows of a song holding its draw."""
    for t, n in ((logits, "logits"), (ids, "ids"), (noise, "noise"), (frame_dev, "frame_dev"),
                 (out, "out")):
        _cuda(t, n)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.shape[0] % 2:
        raise ValueError("logits must be a float32 [2S, V] tensor of row pairs")
    B, V = logits.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=logits.device)
    p = _lib.SampleParams(int(seed) & (2**64 - 1), int(frame), _ptr(frame_dev), int(draw),
                          float(temperature), int(index_base), _ptr(ids), int(valid[0]),
                          int(valid[1]), _ptr(noise))
    check(lib().m3_cfg_topk_draw(_ptr(logits), B // 2, V, logits.stride(0), float(scale),
                                 int(top_k), ctypes.byref(p), _ptr(out), _stream(stream)))
    return out


def rmsnorm_rows(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                 a: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_rmsnorm_rows: bf16 [M, K] -> bf16 [M, K] (the prefill's norm)."""
    for t, n in ((x, "x"), (gamma, "gamma"), (a, "a")):
        _cuda(t, n)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a bf16 [M, K] tensor")
    M, K = x.shape
    if a is None:
        a = torch.empty(M, K, dtype=torch.bfloat16, device=x.device)
    check(lib().m3_rmsnorm_rows(_ptr(x), M, K, x.stride(0), _ptr(gamma), float(eps), _ptr(a),
                                a.stride(0), _stream(stream)))
    return a


def prefill_gemm(packed: torch.Tensor, N: int, K: int, a: torch.Tensor, y: torch.Tensor | None = None,
                 out_dtype: int = OUT_BF16, epi: int = EPI_NONE,
                 residual: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_prefill_gemm: y[M, N] (N/2 for SwiGLU) = epi(a[M, K] . W^T)."""
    for t, n in ((packed, "packed"), (a, "a"), (y, "y"), (residual, "residual")):
        _cuda(t, n)
    M = a.shape[0]
    ncols = N // 2 if epi == EPI_SWIGLU else N
    if y is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
        y = torch.empty(M, ncols, dtype=dt, device=a.device)
    ldr = residual.stride(0) if residual is not None else 0
    check(lib().m3_prefill_gemm(_ptr(packed), N, K, _ptr(a), M, a.stride(0), _ptr(y), y.stride(0),
                                out_dtype, epi, _ptr(residual), ldr, _stream(stream)))
    return y


# ---- decode attention ---------------------------------------------------------
HEAD_DIM = 128


def rope_table(max_pos: int, theta: float = 1e6, device="cuda", stream=None) -> torch.Tensor:
    """m3_rope_table: fp32 [max_pos, 64, 2] (cos, sin of p * theta^(-i/64))."""
    t = torch.empty(max_pos, HEAD_DIM // 2, 2, dtype=torch.float32, device=device)
    check(lib().m3_rope_table(_ptr(t), int(max_pos), HEAD_DIM, float(theta), _stream(stream)))
    return t


def kv_cache(B: int, n_kv: int, max_pos: int, device="cuda") -> tuple[torch.Tensor, torch.Tensor]:
    """Zeroed bf16 K and V caches [B, n_kv, max_pos, 128]."""
    shape = (B, n_kv, max_pos, HEAD_DIM)
    return (torch.zeros(shape, dtype=torch.bfloat16, device=device),
            torch.zeros(shape, dtype=torch.bfloat16, device=device))


def qk_norm_rope(qkv: torch.Tensor, n_q: int, n_kv: int, q_gamma: torch.Tensor,
                 k_gamma: torch.Tensor, rope: torch.Tensor, pos: int, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, eps: float = 1e-6, q_out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """m3_qk_norm_rope: q [B, n_q*128] bf16; k and v written into the caches at pos."""
    for t, n in ((qkv, "qkv"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"), (rope, "rope"),
                 (k_cache, "k_cache"), (v_cache, "v_cache"), (q_out, "q_out")):
        _cuda(t, n)
    B = qkv.shape[0]
    if q_out is None:
        q_out = torch.empty(B, n_q * HEAD_DIM, dtype=torch.bfloat16, device=qkv.device)
    for c in (k_cache, v_cache):
        if c.dim() != 4 or c.shape[0] != B or c.shape[1] != n_kv or c.shape[3] != HEAD_DIM \
                or not c.is_contiguous():
            raise ValueError("caches must be contiguous [B, n_kv, max_pos, 128]")
    check(lib().m3_qk_norm_rope(_ptr(qkv), B, qkv.stride(0), int(n_q), int(n_kv), HEAD_DIM,
                                _ptr(q_gamma), _ptr(k_gamma), float(eps), _ptr(rope), int(pos),
                                _ptr(q_out), q_out.stride(0), _ptr(k_cache), _ptr(v_cache),
                                k_cache.shape[2], _stream(stream)))
    return q_out


def decode_attention_step(qkv: torch.Tensor, n_q: int, n_kv: int, q_gamma: torch.Tensor,
                          k_gamma: torch.Tensor, rope: torch.Tensor, pos: int,
                          k_cache: torch.Tensor, v_cache: torch.Tensor, eps: float = 1e-6,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """m3_decode_attention_step: q/k norm + RoPE at pos (k and v written into
    the caches) and attention over positions <= pos in one launch; out
    [B, n_q*128] bf16."""
    for t, n in ((qkv, "qkv"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"), (rope, "rope"),
                 (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out"), (workspace, "workspace")):
        _cuda(t, n)
    B = qkv.shape[0]
    for c in (k_cache, v_cache):
        if c.dim() != 4 or c.shape[0] != B or c.shape[1] != n_kv or c.shape[3] != HEAD_DIM \
                or not c.is_contiguous():
            raise ValueError("caches must be contiguous [B, n_kv, max_pos, 128]")
    if out is None:
        out = torch.empty(B, n_q * HEAD_DIM, dtype=torch.bfloat16, device=qkv.device)
    need = attention_workspace_bytes(B, n_q, n_kv, pos + 1)
    if workspace is None and need:
        workspace = attention_workspace(B, n_q, n_kv, pos + 1, qkv.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().m3_decode_attention_step(_ptr(qkv), B, qkv.stride(0), int(n_q), int(n_kv), HEAD_DIM,
                                         _ptr(q_gamma), _ptr(k_gamma), float(eps), _ptr(rope),
                                         int(pos), _ptr(k_cache), _ptr(v_cache), k_cache.shape[2],
                                         _ptr(out), out.stride(0), _ptr(workspace), wbytes,
                                         _stream(stream)))
    return out


def attention_workspace_bytes(B: int, n_q: int, n_kv: int, T: int) -> int:
    return int(lib().m3_attention_workspace_bytes(int(B), int(n_q), int(n_kv), int(T)))


def attention_workspace(B: int, n_q: int, n_kv: int, T: int, device="cuda") -> torch.Tensor:
    """A workspace for m3_decode_attention at these sizes."""
    return torch.empty(max(16, attention_workspace_bytes(B, n_q, n_kv, T)), dtype=torch.uint8,
                       device=device)


def decode_attention(q: torch.Tensor, n_q: int, n_kv: int, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, T: int, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_decode_attention: out [B, n_q*128] bf16 over cached positions < T."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out"),
                 (workspace, "workspace")):
        _cuda(t, n)
    B = q.shape[0]
    if out is None:
        out = torch.empty(B, n_q * HEAD_DIM, dtype=torch.bfloat16, device=q.device)
    need = attention_workspace_bytes(B, n_q, n_kv, T)
    if workspace is None and need:
        workspace = attention_workspace(B, n_q, n_kv, T, q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().m3_decode_attention(_ptr(q), B, q.stride(0), int(n_q), int(n_kv), HEAD_DIM,
                                    _ptr(k_cache), _ptr(v_cache), k_cache.shape[2], int(T),
                                    _ptr(out), out.stride(0), _ptr(workspace), wbytes,
                                    _stream(stream)))
    return out


def prefill_qk_norm_rope(qkv: torch.Tensor, S: int, n_q: int, n_kv: int, q_gamma: torch.Tensor,
                         k_gamma: torch.Tensor, rope: torch.Tensor, pos_base: int,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, eps: float = 1e-6,
                         q_out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_prefill_qk_norm_rope: rows [S * P] ordered [s][t]; row (s, t) at
    position pos_base + t of cache s.  Returns q [S * P, n_q * 128]."""
    for t, n in ((qkv, "qkv"), (q_gamma, "q_gamma"), (k_gamma, "k_gamma"), (rope, "rope"),
                 (k_cache, "k_cache"), (v_cache, "v_cache"), (q_out, "q_out")):
        _cuda(t, n)
    R = qkv.shape[0]
    if R % S:
        raise ValueError("rows must be S sequences of equal length")
    if q_out is None:
        q_out = torch.empty(R, n_q * HEAD_DIM, dtype=torch.bfloat16, device=qkv.device)
    check(lib().m3_prefill_qk_norm_rope(_ptr(qkv), S, R // S, qkv.stride(0), int(n_q), int(n_kv),
                                        HEAD_DIM, _ptr(q_gamma), _ptr(k_gamma), float(eps),
                                        _ptr(rope), int(pos_base), _ptr(q_out), q_out.stride(0),
                                        _ptr(k_cache), _ptr(v_cache), k_cache.shape[2],
                                        _stream(stream)))
    return q_out


def prefill_attention(q: torch.Tensor, S: int, n_q: int, n_kv: int, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, pos_base: int, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """m3_prefill_attention: causal attention of rows [S * P] (ordered [s][t])
    over their caches; row (s, t) attends over positions 0 .. pos_base + t."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out"),
                 (workspace, "workspace")):
        _cuda(t, n)
    R = q.shape[0]
    if R % S:
        raise ValueError("rows must be S sequences of equal length")
    P = R // S
    if out is None:
        out = torch.empty(R, n_q * HEAD_DIM, dtype=torch.bfloat16, device=q.device)
    need = int(lib().m3_prefill_attention_workspace_bytes(S, P, int(n_q), int(n_kv), int(pos_base)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().m3_prefill_attention(_ptr(q), S, P, q.stride(0), int(n_q), int(n_kv), HEAD_DIM,
                                     _ptr(k_cache), _ptr(v_cache), k_cache.shape[2], int(pos_base),
                                     _ptr(out), out.stride(0), _ptr(workspace), wbytes,
                                     _stream(stream)))
    return out

