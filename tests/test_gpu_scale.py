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
import transformer_scaled_dot_attn_amd as attn
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


def _structured(seed):
    """A seeded structured mask case: masks that open whole tiles (all-true
    planes or rows, key padding at or off tile edges, the causal rule given
    as a mask, packed documents, windows), with random sizes, broadcast,
    lengths, grouped heads, widths and sometimes a bias."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 6]))
    B = int(rng.integers(1, 4))
    H = int(rng.choice([2, 4, 8]))
    Hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h <= H and H % h == 0]))
    Sq = int(rng.integers(2, 700))
    Skv = Sq if rng.random() < 0.5 else int(rng.integers(Sq, Sq + 6000))
    d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    causal = int(rng.integers(0, 2))
    lens = None if rng.random() < 0.5 else [int(x) for x in rng.integers(1, Skv + 1, size=B)]
    kind = str(rng.choice(["true_plane", "true_row", "pad_edge", "pad_any", "tril", "docs",
                           "window"]))
    if kind == "true_plane":
        mask = np.ones((1, 1, Sq, Skv), dtype=bool)
    elif kind == "true_row":
        mask = np.ones((B if rng.random() < 0.5 else 1, 1, 1, Skv), dtype=bool)
    elif kind in ("pad_edge", "pad_any"):
        hi = max(1, Skv // 2)
        starts = rng.integers(0, hi, size=B)
        if kind == "pad_edge":
            starts = starts // 64 * 64
        mask = W.key_padding_mask([int(x) for x in starts], [Skv] * B, Skv)
    elif kind == "tril":
        mask = np.tril(np.ones((Sq, Skv), dtype=bool), Skv - Sq)[None, None]
    elif kind == "docs":
        cuts = np.sort(rng.choice(np.arange(1, Skv), size=min(3, Skv - 1), replace=False))
        mask = W.document_mask(np.diff(np.concatenate([[0], cuts, [Skv]])).tolist())
        mask = mask[:, :, Skv - Sq:, :]
    else:
        mask = W.window_mask(Skv, int(rng.integers(16, 400)))[:, :, Skv - Sq:, :]
    bias = None
    if rng.random() < 0.25:
        bias = W.random_bias(seed, (1, H, Sq, Skv), "bf16", hide=0.02)
    return B, H, Hkv, Sq, Skv, d, dv, causal, lens, kind, np.ascontiguousarray(mask), bias


@pytest.mark.parametrize("seed", range(400, 430))
def test_random_structured_mask(seed):
    """Structured masks through the prefill's whole-tile paths (tile lists,
    the plain loop, marks made by the pre-pass or by the blocks) against the
    oracle, on random shapes."""
    import torch
    B, H, Hkv, Sq, Skv, d, dv, causal, lens, kind, mask, bias = _structured(seed)
    _say(f"structured {seed}: B{B} H{H}/{Hkv} Sq{Sq} Skv{Skv} d{d}/{dv} causal{causal} "
         f"lens {lens} {kind} {mask.shape} bias {bias is not None}")
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens, Hkv=Hkv, dv=dv)
    tq, tk, tv = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    tl = None if lens is None else torch.as_tensor(np.asarray(lens, np.int32)).to("cuda")
    out = attn.fwd(tq, tk, tv, causal=bool(causal), kv_lens=tl, scale=prob["scale"],
                   mask=W.mask_to_torch(mask),
                   bias=None if bias is None else W.bias_to_torch(bias))
    torch.cuda.synchronize()
    got = W.from_torch(out)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                           mask=mask, bias=bias)
    assert_matches(got, ref, BF16_TOL, lens, Skv, f"s{seed} {kind}")
    assert np.all(got[np.all(ref == 0.0, axis=-1)] == 0.0), "rows without a visible key"
