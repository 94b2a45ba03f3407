"""GPU parity of the reference's draw (DiffSynth-Studio MiniMax-Music3 stage
2: guidance u + 1.5 (c - u) over each song's conditional and unconditional
rows, top-k 50, multinomial sampling as Gumbel-argmax over the survivors)
against the oracle: drawn ids bit-exact given identical fp32 logits, over
every register-run width of the kernel (1..32 columns per thread), ragged
column counts, ties at the top-k boundary, masks, id lists, NaN guidance,
noise overrides and the frame number read from the device."""
import numpy as np
import pytest
import torch

import oracle as O
from autoregressive_audio_lm_amd import m3

pytestmark = pytest.mark.gpu
DEV = "cuda"


def pairs(S, V, seed, scale=2.0):
    return (np.random.default_rng(seed).standard_normal((2 * S, V)) * scale).astype(np.float32)


def same(L, **kw):
    got = m3.cfg_topk_draw(torch.from_numpy(L).to(DEV), **kw).cpu().numpy()
    kw_o = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in kw.items()}
    want = O.cfg_topk_draw(L, **kw_o)
    assert np.array_equal(got, want), (kw, got, want)
    assert np.array_equal(got[0::2], got[1::2])
    return got


@pytest.mark.parametrize("S,V", [(1, 1), (1, 7), (3, 1000), (8, 1024), (2, 1025), (4, 2049),
                                 (5, 5000), (8, 16384), (2, 20000), (1, 32768)])
def test_draw_bit_exact(S, V):
    L = pairs(S, V, V + S)
    for k, seed, frame, draw, T, base in [(50, 0, 0, 0, 1.0, 151675), (1, 7, 12, 3, 0.7, 0),
                                          (V + 3, 2**63 + 5, 1499, 7, 1.3, 5),
                                          (min(V, 700), 11, 3, 1, 1.0, 0)]:
        same(L, scale=1.5, top_k=k, seed=seed, frame=frame, draw=draw, temperature=T,
             index_base=base)


@pytest.mark.parametrize("V", [64, 1000, 16384])
def test_boundary_ties(V):
    """Quantised logits: many columns share the k-th guided value, so the
    survivors are decided by the column order of the ties."""
    rng = np.random.default_rng(V)
    S = 6
    L = (np.round(rng.standard_normal((2 * S, V)) * 2) / 2).astype(np.float32)
    L[1::2] = L[0::2]                  # c == u: the guided value is u itself
    for k in (1, 3, 50):
        for f in range(3):
            same(L, top_k=k, seed=5, frame=f)
    L2 = np.zeros((2 * S, V), np.float32)
    for f in range(3):
        same(L2, top_k=50, seed=9, frame=f)        # every value tied


def test_masks_ids_and_frame_from_device():
    S, V = 4, 16384
    L = pairs(S, V, 3)
    same(L, top_k=50, seed=3, frame=9, index_base=151000, valid=(151675, 160000))
    ids = np.concatenate([[151670], np.arange(151675, 151675 + V - 1)]).astype(np.int32)
    same(L, top_k=50, seed=4, frame=2, ids=torch.from_numpy(ids).to(DEV),
         valid=(151670, 151675 + V))
    fdev = torch.tensor([77], dtype=torch.int32, device=DEV)
    got = m3.cfg_topk_draw(torch.from_numpy(L).to(DEV), seed=4, frame_dev=fdev).cpu().numpy()
    assert np.array_equal(got, O.cfg_topk_draw(L, seed=4, frame=77))
    # every column masked: the first column's id
    got = same(L, top_k=50, index_base=10, valid=(0, 5))
    assert np.all(got == 10)


def test_nan_guidance_and_noise_override():
    S, V = 3, 300
    L = pairs(S, V, 8)
    L[0, 10] = L[1, 10] = np.inf              # inf - inf: song 0 column 10 takes no part
    L[2, :] = L[3, :] = np.inf                # song 1: nothing left
    L[4, 20] = 1e30                           # song 2: a dominant conditional value
    noise = np.random.default_rng(9).gumbel(size=(S, V)).astype(np.float32)
    noise[0, 5] = np.nan
    noise[2, 7] = -np.inf
    for k in (1, 2, 50):
        same(L, top_k=k, seed=1)
        same(L, top_k=k, noise=torch.from_numpy(noise).to(DEV), index_base=3)


def test_back_to_back_calls_independent():
    """Outputs depend only on the call's own inputs (no state carried in the
    library between calls of different shapes)."""
    big = pairs(8, 16384, 21)
    small = pairs(2, 1000, 22)
    a1 = same(big, top_k=50, seed=2, frame=1)
    same(small, top_k=5, seed=2, frame=1)
    a2 = same(big, top_k=50, seed=2, frame=1)
    assert np.array_equal(a1, a2)


@pytest.mark.parametrize("k", [1000, 1024, 1025, 4000])
def test_k_near_the_compaction_bound(k):
    """k around the 1024 keys the kernel compacts into LDS: both the
    compacted and the in-register finish give the oracle's draws."""
    L = pairs(4, 16384, 31 + k)
    for f in range(3):
        same(L, top_k=k, seed=6, frame=f)
    Lq = (np.round(L * 4) / 4).astype(np.float32)        # ties straddle the bound
    for f in range(3):
        same(Lq, top_k=k, seed=6, frame=f)
