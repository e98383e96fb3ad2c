"""Long contexts and random combinations of every option, on the GPU.

Long contexts exercise the large-offset paths: a 16384-token causal prefill
(checked on sampled rows, each against the oracle over exactly the keys its
position sees), a decode over a 131072-key cache, and a 300-token chunk
against a 65536-key cache (the most key-range splits).  The combination sweep
draws 40 seeded problems over dtype, batch, heads, K/V grouping, query and key
lengths (Sq = 1 included), head size, causal flag, valid lengths and
allowed-mask shapes, and compares each with the oracle element by element.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, gpu_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_prefill16k_sampled_rows():
    """Row p of a causal prefill equals attention of query p over keys 0..p
    (reading 3 with Sq = Skv); the oracle computes only the sampled rows."""
    B, H, Hkv, S, d = 1, 4, 2, 16384, 128
    _say("prefill 16384 sampled rows")
    prob = W.random_problem(201, B, H, S, S, d, "bf16", Hkv=Hkv)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    for p in (0, 1, 255, 256, 4097, 8191, 12000, 16383):
        q = prob["q"][:, :, p:p + 1]
        ref = oracle.attention(q, prob["k"][:, :, :p + 1], prob["v"][:, :, :p + 1],
                               prob["scale"], 1)
        assert_matches(got[:, :, p:p + 1], ref, BF16_TOL, what=f"row {p}")


def test_decode_128k_cache():
    B, H, Hkv, Skv, d = 2, 8, 1, 131072, 128
    _say("decode over a 131072-key cache")
    lens = [131072, 70001]
    prob = W.random_problem(202, B, H, 1, Skv, d, "bf16", lens, Hkv=Hkv)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    assert_matches(got, ref, BF16_TOL, lens, Skv, "decode 128k")


def test_chunk_against_64k_cache():
    B, H, S, c, d = 1, 2, 65536, 300, 128
    _say("chunk of 300 queries against 65536 keys")
    prob = W.random_problem(203, B, H, c, S, d, "bf16")
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    rows = [0, 1, 150, 299]
    for i in rows:
        p = S - c + i  # bottom-right alignment
        ref = oracle.attention(prob["q"][:, :, i:i + 1], prob["k"][:, :, :p + 1],
                               prob["v"][:, :, :p + 1], prob["scale"], 1)
        assert_matches(got[:, :, i:i + 1], ref, BF16_TOL, what=f"chunk row {i}")


def _combination(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5]))
    dt = "f32" if rng.random() < 0.25 else "bf16"
    B = int(rng.integers(1, 4))
    H = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h <= H and H % h == 0]))
    Sq = 1 if rng.random() < 0.3 else int(rng.integers(2, 300))
    Skv = int(rng.integers(Sq, Sq + 900))
    d = int(rng.choice([64, 128])) if dt == "bf16" else int(rng.integers(1, 129))
    causal = int(rng.integers(0, 2))
    lens = None if rng.random() < 0.4 else [int(x) for x in rng.integers(-5, Skv + 20, size=B)]
    shape = None
    if rng.random() < 0.5:
        shape = (B if rng.random() < 0.5 else 1, H if rng.random() < 0.5 else 1,
                 Sq if rng.random() < 0.6 else 1, Skv)
    density = float(rng.uniform(0.05, 0.95))
    return dt, B, H, Hkv, Sq, Skv, d, causal, lens, shape, density


@pytest.mark.parametrize("seed", range(300, 340))
def test_random_combination(seed):
    dt, B, H, Hkv, Sq, Skv, d, causal, lens, shape, density = _combination(seed)
    _say(f"combination {seed}: {dt} B{B} H{H}/{Hkv} Sq{Sq} Skv{Skv} d{d} causal{causal} "
         f"lens {lens} mask {shape}")
    prob = W.random_problem(seed, B, H, Sq, Skv, d, dt, lens, Hkv=Hkv)
    mask = None if shape is None else W.random_mask(seed, shape, density)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                     mask=None if mask is None else W.mask_to_torch(mask))
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, clamped,
                           mask=mask)
    assert_matches(got, ref, F32_TOL if dt == "f32" else BF16_TOL, clamped, Skv, f"c{seed}")
    assert np.all(got[np.all(ref == 0.0, axis=-1)] == 0.0), "rows without a visible key"
