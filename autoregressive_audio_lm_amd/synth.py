"""Seeded synthetic inputs (weights, gammas, activations) shared by the tests,
the benchmark and the smoke check.

This module holds none of the decode arithmetic: it only draws numbers.
Weights ~ N(0, 0.02) and activations ~ N(0, 1) as bf16, norm gammas
1 + N(0, 0.1) as fp32, following the benchmark shapes.  Values come from
torch's generator on the requested device; each tensor has its own seed
derived from (model seed, layer, tensor id), so any tensor can be regenerated
alone.
"""
from __future__ import annotations

import numpy as np
import torch

W_STD = 0.02


def tensor_seed(base: int, layer: int, tid: int) -> int:
    return (int(base) * 1000003 + int(layer) * 1009 + int(tid)) & 0x7FFFFFFFFFFF


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """bf16 tensor of N(0, std^2) draws (rounded by torch's bf16 cast)."""
    t = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def gamma_f32(n: int, seed: int, device="cpu") -> torch.Tensor:
    t = torch.randn(n, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(0.1).add_(1.0)


def uniform_f32(shape, seed: int, lo: float, hi: float, device="cpu") -> torch.Tensor:
    t = torch.rand(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


# tensor ids
_T = dict(qkv=1, o=2, gate=3, up=4, down=5, attn_norm=6, ffn_norm=7, q_norm=8, k_norm=9)


def make_model(cfg: dict, fmt_body: int, fmt_lm: int, fmt_depth: int, seed: int = 0,
               device="cpu", n_layers: int | None = None) -> dict:
    """All weights of one decode frame as torch tensors on `device` (bf16
    sources; int8 formats are quantised later by whoever consumes them).
    Gate and up are separate [F, H] tensors."""
    H, F = cfg["H"], cfg["F"]
    nq = cfg["n_heads"] * cfg["head_dim"]
    nkv = cfg["n_kv_heads"] * cfg["head_dim"]
    D, Fd = cfg["D"], cfg["Fd"]
    dq = cfg["d_heads"] * cfg["d_head_dim"]
    L = cfg["n_layers"] if n_layers is None else n_layers

    def layer(li, h, q_out, kv_out, f, base):
        return {
            "qkv": normal_bf16((q_out + 2 * kv_out, h), tensor_seed(base, li, _T["qkv"]), W_STD, device),
            "o": normal_bf16((h, q_out), tensor_seed(base, li, _T["o"]), W_STD, device),
            "gate": normal_bf16((f, h), tensor_seed(base, li, _T["gate"]), W_STD, device),
            "up": normal_bf16((f, h), tensor_seed(base, li, _T["up"]), W_STD, device),
            "down": normal_bf16((h, f), tensor_seed(base, li, _T["down"]), W_STD, device),
            "attn_norm": gamma_f32(h, tensor_seed(base, li, _T["attn_norm"]), device),
            "ffn_norm": gamma_f32(h, tensor_seed(base, li, _T["ffn_norm"]), device),
            # per-head q/k RMSNorm gammas (decode attention)
            "q_norm": gamma_f32(cfg["head_dim"], tensor_seed(base, li, _T["q_norm"]), device),
            "k_norm": gamma_f32(cfg["head_dim"], tensor_seed(base, li, _T["k_norm"]), device),
        }

    md = {"cfg": dict(cfg), "fmt_body": fmt_body, "fmt_lm": fmt_lm, "fmt_depth": fmt_depth}
    md["layers"] = [layer(li, H, nq, nkv, F, seed) for li in range(L)]
    md["final_norm"] = gamma_f32(H, tensor_seed(seed, 900, 1), device)
    md["lm_head"] = normal_bf16((cfg["V0"], H), tensor_seed(seed, 900, 2), W_STD, device)
    # the lm_head row of the end token (used when a frame draws it)
    md["lm_end"] = normal_bf16((1, H), tensor_seed(seed, 900, 5), W_STD, device)
    dseed = seed + 7777
    md["d_layers"] = [layer(li, D, dq, dq, Fd, dseed) for li in range(cfg["d_layers"])]
    md["d_final_norm"] = gamma_f32(D, tensor_seed(dseed, 900, 1), device)
    md["p_in"] = normal_bf16((D, H), tensor_seed(dseed, 900, 3), W_STD, device)
    md["emb1"] = normal_bf16((cfg["V0"], D), tensor_seed(dseed, 900, 4), W_STD, device)
    nsteps = cfg["n_codebooks"] - 1
    md["emb"] = [normal_bf16((cfg["code_vocab"], D), tensor_seed(dseed, 910 + j, 4), W_STD, device)
                 for j in range(2, nsteps + 1)]
    md["heads"] = [normal_bf16((cfg["code_vocab"], D), tensor_seed(dseed, 920 + j, 5), W_STD, device)
                   for j in range(1, nsteps + 1)]
    md["tok_emb_audio"] = normal_bf16((cfg["V0"], H), tensor_seed(seed, 930, 6), W_STD, device)
    md["audio_emb"] = [normal_bf16((cfg["code_vocab"], H), tensor_seed(seed, 940 + j, 7), W_STD, device)
                       for j in range(1, nsteps + 1)]
    return md


def model_to_numpy(md: dict) -> dict:
    """Host copy of a model dict: bf16 -> uint16 bits, fp32 -> float32."""
    def cv(v):
        if isinstance(v, torch.Tensor):
            return bits(v) if v.dtype == torch.bfloat16 else v.detach().cpu().numpy()
        if isinstance(v, list):
            return [cv(x) for x in v]
        if isinstance(v, dict):
            return {k: cv(x) for k, x in v.items()}
        return v
    return cv(md)


def activations(B: int, K: int, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """[B, K] bf16 rows, each row from its own seed (seed + 100 + b)."""
    rows = [normal_bf16((1, K), seed + 100 + b, std, device) for b in range(B)]
    return torch.cat(rows, 0)
