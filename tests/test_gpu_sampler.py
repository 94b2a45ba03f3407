"""GPU parity of the Philox Gumbel-argmax sampler (bit-exact against the
oracle given identical fp32 logits) and of the sliced lm_head (diffusers
issue #14486, item 3: slicing the lm_head to the sampleable rows is identical
to masking the other rows to -inf)."""
import numpy as np
import pytest
import torch

import oracle as O
import parity as P
from autoregressive_audio_lm_amd import m3, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def logits_np(B, V, seed, scale=3.0):
    return (np.random.default_rng(seed).standard_normal((B, V)) * scale).astype(np.float32)


@pytest.mark.parametrize("B,V,base", [(1, 1, 0), (1, 3, 7), (5, 1000, 0), (16, 1024, 0),
                                      (3, 1025, 5), (16, 16384, 151675), (2, 20000, 1),
                                      (64, 333, 2)])
def test_argmax_bit_exact(B, V, base):
    L = logits_np(B, V, V + B)
    Ld = torch.from_numpy(L).to(DEV)
    for seed, frame, draw, T in [(0, 0, 0, 1.0), (7, 12, 3, 0.7), (2**63 + 5, 1499, 7, 1.3)]:
        got = m3.gumbel_argmax(Ld, seed=seed, frame=frame, draw=draw, temperature=T,
                               index_base=base).cpu().numpy()
        want = O.gumbel_argmax(L, seed=seed, frame=frame, draw=draw, temperature=T, index_base=base)
        assert np.array_equal(got, want), (seed, frame, draw)


def test_argmax_mask_ids_and_frame_from_device():
    B, V = 6, 5000
    L = logits_np(B, V, 1)
    Ld = torch.from_numpy(L).to(DEV)
    got = m3.gumbel_argmax(Ld, seed=3, frame=9, index_base=151000, valid=(151675, 153000)).cpu().numpy()
    want = O.gumbel_argmax(L, seed=3, frame=9, index_base=151000, valid=(151675, 153000))
    assert np.array_equal(got, want) and np.all((got >= 151675) & (got < 153000))
    ids = np.random.default_rng(2).permutation(200000)[:V].astype(np.int32)
    got = m3.gumbel_argmax(Ld, seed=4, frame=2, ids=torch.from_numpy(ids).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.gumbel_argmax(L, seed=4, frame=2, ids=ids))
    fdev = torch.tensor([77], dtype=torch.int32, device=DEV)
    got = m3.gumbel_argmax(Ld, seed=4, frame=0, frame_dev=fdev).cpu().numpy()
    assert np.array_equal(got, O.gumbel_argmax(L, seed=4, frame=77))


def test_argmax_ties_nan_masked_rows():
    V = 64
    L = np.zeros((4, V), np.float32)
    noise = np.zeros((4, V), np.float32)
    noise[0, [9, 40]] = 2.0
    noise[1, [5, 6]] = np.nan
    noise[2, :] = -np.inf
    L[3, :] = -np.inf
    got = m3.gumbel_argmax(torch.from_numpy(L).to(DEV), noise=torch.from_numpy(noise).to(DEV),
                           index_base=100).cpu().numpy()
    want = O.gumbel_argmax(L, noise=noise, index_base=100)
    assert np.array_equal(got, want) and list(got) == [109, 105, 100, 100]


def test_sampling_law_on_gpu():
    """200k draws at V = 32 reproduce softmax(l/T) within L1 <= 0.02."""
    V, B, frames = 32, 1000, 200
    lg = (np.random.default_rng(5).standard_normal(V) * 1.5).astype(np.float32)
    Ld = torch.from_numpy(np.repeat(lg[None], B, 0)).to(DEV)
    counts = torch.zeros(V, dtype=torch.int64, device=DEV)
    out = torch.empty(B, dtype=torch.int32, device=DEV)
    for f in range(frames):
        m3.gumbel_argmax(Ld, seed=11, frame=f, out=out)
        counts += torch.bincount(out.long(), minlength=V)
    p = np.exp(lg - lg.max())
    p /= p.sum()
    l1 = np.abs(counts.cpu().numpy() / (B * frames) - p).sum()
    assert l1 <= 0.02, l1


# ----------------------------------------------------------- lm_head ------
@pytest.mark.parametrize("fmt,B", [(0, 16), (0, 1), (1, 6)])
def test_sliced_lmhead_equals_masked_full(fmt, B):
    """Full bf16 vocab [200000, 4096] vs the 16384 reachable rows: identical
    logits for the slice rows, identical draws; sampled rows vs the oracle."""
    H, Vfull, base, V0 = 4096, 200000, 151675, 16384
    Wf = synth.normal_bf16((Vfull, H), 700, 0.02, DEV)
    x = synth.activations(B, H, 710, DEV)
    g = synth.gamma_f32(H, 711, DEV)
    pk_full = m3.pack(fmt, Wf)
    Ws = Wf[base:base + V0].contiguous()
    pk_slice = m3.pack(fmt, Ws)
    lf = m3.lmhead_sliced(fmt, pk_full, Vfull, H, x, g)
    ls = m3.lmhead_sliced(fmt, pk_slice, V0, H, x, g)
    torch.cuda.synchronize()
    assert torch.equal(lf[:, base:base + V0], ls)
    del pk_full
    for frame in range(4):
        a = m3.gumbel_argmax(lf, seed=13, frame=frame, index_base=0, valid=(base, base + V0))
        b = m3.gumbel_argmax(ls, seed=13, frame=frame, index_base=base)
        assert torch.equal(a, b)
    # sampled rows against the oracle (one by one)
    rows = np.sort(np.random.default_rng(3).choice(V0, 96, replace=False))
    Wrows = synth.bits(Ws[torch.from_numpy(rows).to(DEV)])
    a = O.rmsnorm(synth.bits(x), g.cpu().numpy(), 1e-6)
    y_ex = O.gemv(O.Matrix(Wrows, fmt), a)
    P.check_f32(ls.cpu().numpy()[:, rows], y_ex)
