"""Grouped key/value heads (GQA / MQA) on the GPU against the CPU oracle.

Query head h reads K/V head h // (H // H_kv).  Every kernel family is run
with K/V heads in {1, 2, ..., H} on ragged shapes and compared element by
element with the oracle; prefill and fp32 results must also equal, bit for
bit, the multi-head call on K and V expanded with repeat_interleave (the
kernels' per-head arithmetic does not depend on where a head's K/V lives).
The full-size grouped workloads run in the benchmark's launch configuration
and are compared on sampled (batch, head) slices.  Grouped bf16 decode
without a mask runs the stream kernel, whose wave shares cross pair and batch
boundaries; its edge cases (empty caches, more than 64 batch items, fewer
tiles than one wave's floor, two head groups per K/V head) have cases of
their own.
"""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, check_workload_full, gpu_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


CASES = [
    # seed, dtype, B, H, Hkv, Sq, Skv, d, causal, kv_lens
    (41, "f32", 2, 4, 1, 70, 70, 32, 1, [70, 33]),
    (42, "f32", 1, 6, 3, 1, 150, 128, 0, None),
    (43, "bf16", 2, 8, 2, 300, 300, 128, 1, [300, 129]),
    (44, "bf16", 1, 8, 1, 200, 200, 64, 1, None),
    (45, "bf16", 2, 4, 4, 130, 260, 128, 1, [260, 90]),
    (46, "bf16", 1, 16, 4, 64, 64, 128, 0, None),
    (47, "bf16", 3, 8, 2, 1, 1000, 128, 0, [1000, 1, 0]),
    (48, "bf16", 2, 16, 1, 1, 700, 64, 0, [700, 65]),
    (49, "bf16", 2, 32, 8, 1, 2100, 128, 0, [2100, 777]),
    (50, "bf16", 1, 12, 6, 1, 513, 128, 0, None),
    (51, "bf16", 2, 24, 3, 1, 300, 128, 0, [300, 17]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_gqa_shapes(case):
    seed, dtype, B, H, Hkv, Sq, Skv, d, causal, lens = case
    _say("gqa case", case)
    prob = W.random_problem(seed, B, H, Sq, Skv, d, dtype, lens, Hkv=Hkv)
    q, k, v, scale = prob["q"], prob["k"], prob["v"], prob["scale"]
    got, _ = gpu_run(q, k, v, scale, causal, lens)
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(q, k, v, scale, causal, clamped)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    assert_matches(got, ref, tol, clamped, Skv, f"gqa {case}")
    # the multi-head call on expanded K/V
    g = H // Hkv
    ke, ve = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    exp, _ = gpu_run(q, ke, ve, scale, causal, lens)
    if Sq > 1 or dtype == "f32":
        assert np.array_equal(got, exp), f"gqa {case}: differs from the expanded MHA call"
    else:
        assert_matches(got, exp, BF16_TOL, clamped, Skv, f"gqa {case} vs expanded")


# Stream decode (bf16, Sq = 1, 4 or more query heads per K/V head, no mask):
# a fixed grid of waves shares all key tiles of all (batch item, K/V head,
# head group) pairs equally, at least 16 tiles of 32 keys per wave.
STREAM = [
    # name, B, H, Hkv, Skv, d, lengths (None: all Skv; "rand:seed": drawn in [0, Skv])
    ("one key", 1, 4, 1, 1, 128, None),
    ("one tile each", 3, 8, 2, 32, 128, [32, 1, 31]),
    ("fewer tiles than the floor", 2, 16, 4, 200, 64, [200, 0]),
    ("short and empty caches, B 70", 70, 16, 2, 300, 128, "rand:61"),
    ("B 200 groups of 4", 200, 8, 2, 600, 128, "rand:62"),
    ("tile edges", 6, 32, 8, 1100, 128, [1024, 1025, 1023, 992, 33, 64]),
    ("64 heads per K/V head", 3, 64, 1, 1500, 128, [1500, 31, 0]),
    ("48 heads per K/V head", 2, 48, 1, 2500, 128, [2500, 1999]),
    ("d 64 long", 5, 16, 4, 4000, 64, "rand:63"),
    ("every cache empty", 3, 8, 2, 500, 128, [0, 0, 0]),
    ("B 1030, 17 batch items per lane", 1030, 8, 2, 100, 128, "rand:64"),
    ("B 4500 multi-head, 71 per lane", 4500, 2, 2, 40, 64, "rand:65"),
    # hundreds of partials per (b, K/V head): the combine's groups take
    # several rounds of slots, with a ragged last round
    ("one long cache, 8 K/V heads", 1, 32, 8, 32768, 128, None),
    ("one long cache d 64", 1, 16, 2, 40000, 64, [39999]),
]


def _stream_lens(spec, B, Skv):
    if spec is None or not isinstance(spec, str):
        return spec
    rng = np.random.default_rng(int(spec.split(":")[1]))
    lens = rng.integers(0, Skv + 1, size=B)
    lens[rng.random(B) < 0.2] = 0  # runs of empty caches
    return [int(x) for x in lens]


@pytest.mark.parametrize("case", STREAM, ids=lambda c: c[0].replace(" ", "_"))
def test_stream_decode_matches_oracle(case):
    name, B, H, Hkv, Skv, d, spec = case
    lens = _stream_lens(spec, B, Skv)
    _say(f"stream decode {name}: B{B} H{H}/{Hkv} Skv{Skv} d{d}")
    prob = W.random_problem(sum(map(ord, name)), B, H, 1, Skv, d, "bf16", lens, Hkv=Hkv)
    got, t1 = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    assert_matches(got, ref, BF16_TOL, lens, Skv, name)
    if lens is not None:
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(got[b] == 0.0), f"{name}: empty cache {b} not zero"
    # a fixed schedule: the same call gives the same bits
    _, t2 = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    import torch
    assert torch.equal(t1, t2)


def test_gqa_rejects_uneven_groups():
    import torch
    q = torch.zeros(1, 6, 4, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="multiple"):
        attn.fwd(q, k, k)
    lib = attn.library()
    out = torch.empty_like(q)
    rc = lib.attn_fwd_gqa(q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), 1, 6, 4, 4,
                          4, 64, 0.125, 1, None, attn.BF16, None)
    assert rc == attn.E_SHAPE


def test_workload_gqa_prefill2048_full():
    check_workload_full(W.WORKLOADS["gqa_prefill2048_bf16"], say=print)


@pytest.mark.parametrize("name", ["gqa_decode8192_bf16", "mqa_decode8192_bf16"])
def test_workload_grouped_decode_full(name):
    check_workload_full(W.WORKLOADS[name], say=print)
