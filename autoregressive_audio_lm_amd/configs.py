"""Model shapes of the decode path (plain data, no arithmetic).

Body: Qwen3-shaped, hidden 4096, 36 layers, 32 query heads and 8 KV heads of
128 (DiffSynth-Studio MiniMax-Music3 article, model overview).  FFN width
12288 is an assumption (the pages do not print it).  Depth decoder: 4 layers,
16 heads (same overview); hidden 2048 and FFN 5632 are assumptions.  The audio
codes occupy vocab ids [151675, 151675 + 16384); 8 codebooks of which 7 are
drawn by the depth decoder with 1024 codes each (same article, stage 2).
"""
from __future__ import annotations

import copy

FULL = dict(
    name="frame-full",
    H=4096, n_layers=36, n_heads=32, n_kv_heads=8, head_dim=128, F=12288,
    vocab=200000, vocab_base=151675, V0=16384, end_token=151670,
    D=2048, d_layers=4, d_heads=16, d_head_dim=128, Fd=5632,
    n_codebooks=8, code_vocab=1024, eps=1e-6,
)

# A structurally identical model the oracle runs in seconds: several 16-row
# tiles per matrix, ragged row counts (V0, code_vocab) and a ragged K (F).
SMALL = dict(
    name="frame-small",
    H=512, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=128, F=1008,
    vocab=200000, vocab_base=151675, V0=1000, end_token=151670,
    D=256, d_layers=2, d_heads=2, d_head_dim=128, Fd=384,
    n_codebooks=8, code_vocab=104, eps=1e-6,
)

# weight formats (mirror of the C enum)
BF16, I8ROW, I8G128, FP8ROW = 0, 1, 2, 3

# Frame presets: (body, lm_head, depth) formats.
PRESETS = {
    "A": dict(fmt_body=BF16, fmt_lm=BF16, fmt_depth=I8G128),    # bf16 body (headline)
    "B": dict(fmt_body=I8ROW, fmt_lm=I8ROW, fmt_depth=I8G128),  # int8 everywhere
    # fp8 (OCP E4M3, one scale per row) body and lm_head: the fp8 weight-only
    # variant, an assumed format (the pages list fp8 only as a result on
    # another stack)
    "C": dict(fmt_body=FP8ROW, fmt_lm=FP8ROW, fmt_depth=I8G128),
}


def config(name: str = "frame-full", **over) -> dict:
    base = {"frame-full": FULL, "frame-small": SMALL}[name]
    c = copy.deepcopy(base)
    c.update(over)
    return c
