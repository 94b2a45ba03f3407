"""The allocation-free Gumbel-argmax draw (m3_gumbel_argmax_noalloc: the
library's fixed per-device scratch in place of a caller workspace, for
callers that cannot allocate) against the draw with a caller workspace
(m3_gumbel_argmax), through the C ABI: identical ids on consecutive calls
that reuse the scratch, the second with a smaller input, with masks, id
lists, noise overrides and the frame counter read on the device."""
import pytest
import torch

from autoregressive_audio_lm_amd import _lib, m3

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _logits(B, V, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(B, V, device=DEV, generator=g) * 3.0


def test_noalloc_draw_equals_workspace_draw():
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    cases = [  # (B, V, keyword arguments); the second and later calls are smaller
        (64, 300000, dict(seed=7, frame=3, draw=0, index_base=151675, valid=(151700, 400000))),
        (3, 1000, dict(seed=9, frame=11, draw=5)),
        (16, 16384, dict(seed=1, draw=2, temperature=0.7)),
        (1, 1, dict(seed=2)),
    ]
    with torch.cuda.stream(s):
        frame_dev = torch.tensor([41], dtype=torch.int32, device=DEV)
        for i, (B, V, kw) in enumerate(cases):
            lg = _logits(B, V, 100 + i)
            want = m3.gumbel_argmax(lg, stream=s, **kw)
            out = torch.full((B,), -1, dtype=torch.int32, device=DEV)
            got = m3.gumbel_argmax_noalloc(lg, out=out, stream=s, **kw)
            s.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.equal(got, want), (B, V)
        # id list, noise override and the frame number read on the device
        B, V = 5, 3000
        lg = _logits(B, V, 200)
        ids = torch.randperm(100000, device=DEV)[:V].to(torch.int32)
        noise = _logits(B, V, 201)
        for kw in (dict(ids=ids), dict(noise=noise), dict(frame_dev=frame_dev, draw=4)):
            want = m3.gumbel_argmax(lg, seed=3, stream=s, **kw)
            got = m3.gumbel_argmax_noalloc(lg, seed=3, stream=s, **kw)
            s.synchronize()
            assert torch.equal(got, want)
    # a draw whose winners exceed the scratch is refused before anything runs
    big = torch.empty(2, 1, device=DEV)
    with pytest.raises(_lib.M3ValueError):
        _lib.check(_lib.lib().m3_gumbel_argmax_noalloc(
            m3._ptr(big), 16, 1 << 24, 1 << 24,
            __import__("ctypes").byref(_lib.SampleParams(0, 0, None, 0, 1.0, 0, None, 0, 0, None)),
            m3._ptr(big), m3._stream(None)))
