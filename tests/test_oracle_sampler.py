"""Pins of the oracle's sampler: Philox-4x32-10 against rocRAND's
implementation of the published generator, the fp32 log against float64 log,
the uniform map's exactness, Gumbel moments, the sampling law of
Gumbel-argmax (diffusers issue #14486, item 3: identical distribution to
softmax + multinomial, L1 about 0.015 over 200k draws), masking, ties and
non-finite ordering.  CPU only."""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND pin helper")
    exe = str(tmp_path_factory.mktemp("pin") / "philox_pin")
    subprocess.check_call([hipcc, "-O1", "-o", exe, os.path.join(HERE, "pins", "philox_rocrand.cpp")],
                          cwd="/tmp")

    def run(tuples):
        inp = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in tuples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(oracle, rocrand_philox):
    rng = np.random.default_rng(20)
    # the helper addresses counter words (c0, c1) through a 64-bit offset of
    # 4*(c1:c0) numbers, so c1 stays below 2^30 (c1 is the batch row here)
    tuples = [(0, 0, 0, 0, 0), (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1)]
    for _ in range(300):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(v) for v in rng.integers(0, 2**32, 4, dtype=np.uint64)]
        c[1] &= 2**30 - 1
        tuples.append((seed,) + tuple(c))
    ref = rocrand_philox(tuples)
    for t, r in zip(tuples, ref):
        seed = t[0]
        ours = oracle.philox4x32_10(t[1:], [seed & 0xFFFFFFFF, seed >> 32])
        assert tuple(int(v) for v in ours) == r, t


def test_logf_accuracy_vs_float64(oracle):
    rng = np.random.default_rng(21)
    xs = np.concatenate([
        rng.uniform(0, 1, 20000), rng.uniform(0, 20, 20000),
        np.exp(rng.uniform(-85, 85, 20000)),
        [1.0, 2.0, 0.5, 1.4142135, 1.4142137, 0.70710677, 2.0**-25, 1 - 2.0**-24, 17.33],
    ]).astype(np.float32)
    xs = xs[xs > np.float32(1.2e-38)]
    worst = 0.0
    for x in xs:
        got = oracle.logf(x)
        ref = math.log(float(x))
        ulp = np.spacing(np.float32(abs(ref))) if ref != 0 else np.float32(1e-45)
        worst = max(worst, abs(got - ref) / float(ulp))
    assert oracle.logf(1.0) == 0.0
    assert worst <= 4.0, worst


def test_uniform_is_exact_and_open(oracle):
    # cells of width 2^-23 over (0, 1), one value per cell at its midpoint:
    # the first and last cell, symmetry u(k) + u(last - k) = 1, monotone steps
    lo = oracle.uniform_from_word(0)
    hi = oracle.uniform_from_word(2**32 - 1)
    assert lo == 2.0**-24 and hi == 1.0 - 2.0**-24
    rng = np.random.default_rng(25)
    for k in rng.integers(0, 2**23, 2000):
        k = int(k)
        u = oracle.uniform_from_word(k << 9)
        assert 0.0 < u < 1.0
        assert u + oracle.uniform_from_word((2**23 - 1 - k) << 9) == 1.0
        assert oracle.uniform_from_word((k << 9) | 511) == u          # low 9 bits unused
        if k + 1 < 2**23:
            assert oracle.uniform_from_word((k + 1) << 9) - u == 2.0**-23


def test_gumbel_moments(oracle):
    n = 400000
    g = np.array([oracle.gumbel(123, r % 64, r // 64, 0, 7) for r in range(n)], dtype=np.float64)
    em = 0.5772156649015329
    var = math.pi ** 2 / 6
    se_mean = math.sqrt(var / n)
    assert abs(g.mean() - em) < 5 * se_mean
    # variance of the sample variance of a Gumbel: (mu4 - sigma^4)/n, mu4 = 27/5 sigma^4
    se_var = math.sqrt((5.4 - 1.0) * var * var / n)
    assert abs(g.var() - var) < 5 * se_var


def _softmax(l):
    z = l - l.max()
    e = np.exp(z)
    return e / e.sum()


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_sampling_law_l1(oracle, T):
    """200k Gumbel-argmax draws vs softmax(l/T): L1 <= 0.02 at V = 32."""
    rng = np.random.default_rng(22)
    V = 32
    logits = (rng.standard_normal(V) * 1.5).astype(np.float32)
    B, frames = 1000, 200
    L = np.repeat(logits[None, :], B, 0)
    counts = np.zeros(V)
    for f in range(frames):
        ids = oracle.gumbel_argmax(L, seed=99, frame=f, draw=0, temperature=T)
        counts += np.bincount(ids, minlength=V)
    p = _softmax(logits.astype(np.float64) / T)
    l1 = np.abs(counts / counts.sum() - p).sum()
    assert l1 <= 0.02, l1


def test_masking_and_single_finite(oracle):
    rng = np.random.default_rng(23)
    V = 64
    L = rng.standard_normal((16, V)).astype(np.float32)
    # ids 100..163, valid [120, 140)
    for f in range(50):
        ids = oracle.gumbel_argmax(L, seed=5, frame=f, index_base=100, valid=(120, 140))
        assert np.all((ids >= 120) & (ids < 140))
    L2 = np.full((4, V), -np.inf, np.float32)
    L2[:, 17] = 3.0
    for f in range(20):
        assert np.all(oracle.gumbel_argmax(L2, seed=1, frame=f) == 17)


def test_ties_nan_and_all_masked(oracle):
    V = 8
    L = np.zeros((3, V), np.float32)
    noise = np.zeros((3, V), np.float32)
    noise[0, [2, 5]] = 1.0               # tie between 2 and 5 -> 2
    noise[1, 4] = np.nan                 # NaN ranks above everything
    noise[1, 6] = np.nan                 # first NaN wins
    noise[2, :] = -np.inf                # all -inf -> first id
    out = oracle.gumbel_argmax(L, noise=noise, index_base=10)
    assert list(out) == [12, 14, 10]
    full_mask = oracle.gumbel_argmax(np.zeros((1, V), np.float32), index_base=0, valid=(100, 200))
    assert full_mask[0] == 0


def test_sliced_equals_masked_full(oracle):
    """Sampling a contiguous slice with noise keyed by absolute id equals
    sampling the full vocabulary with every other row masked to -inf."""
    rng = np.random.default_rng(24)
    Vfull, base, V0 = 3000, 1675, 640
    full = rng.standard_normal((6, Vfull)).astype(np.float32)
    for f in range(30):
        a = oracle.gumbel_argmax(full, seed=11, frame=f, index_base=0, valid=(base, base + V0))
        b = oracle.gumbel_argmax(np.ascontiguousarray(full[:, base:base + V0]), seed=11, frame=f,
                                 index_base=base, valid=(base, base + V0))
        c = oracle.gumbel_argmax(np.ascontiguousarray(full[:, base:base + V0]), seed=11, frame=f,
                                 ids=np.arange(base, base + V0, dtype=np.int32))
        assert np.array_equal(a, b) and np.array_equal(b, c)


def test_noise_keyed_by_row_frame_draw(oracle):
    g = {(r, f, d): float(oracle.gumbel(3, r, f, d, 151680)) for r in range(3) for f in range(3) for d in range(3)}
    assert len(set(g.values())) == 27
    assert float(oracle.gumbel(3, 1, 2, 1, 151680)) == g[(1, 2, 1)]
