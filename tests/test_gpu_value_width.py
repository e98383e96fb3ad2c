"""A value width d_v different from d on the GPU (every kernel family).

softmax(scale Q K^T) V needs V's rows to line up with K's, not its width to
match d ("Attention from Scratch", KubeDojo module 1.4.3, Part 2, whose
worked example has d_k = 4 and d_v = 2).  The worked example runs at its own
shape against the printed values and the oracle; random shapes with every
width class on each side, with the causal rule, valid lengths, grouped heads
and masks, are compared with the oracle.  The bf16 kernels take d and d_v
each in {64, 128} (prefill, key-range splits, decode, with masks, biases and
grouped heads) and refuse other widths.
"""
import numpy as np
import pytest

import golden_io
import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, gpu_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_worked_example_at_its_own_shape():
    g = golden_io.load("p3_unmasked_3tok_dk4_dv2.txt")
    q, k, v = (g[x][None, None].astype(np.float32) for x in ("q", "k", "v"))
    assert q.shape[-1] == 4 and v.shape[-1] == 2
    scale = float(np.float32(g["scale"]))
    got, _ = gpu_run(q, k, v, scale, g["causal"])
    assert got.shape == (1, 1, 3, 2)
    ref = oracle.attention(q, k, v, scale, g["causal"])
    assert_matches(got, ref, F32_TOL, what="worked example")
    oexp, otol = g["out"]
    assert np.all(np.abs(got[0, 0] - oexp) <= otol), got[0, 0]


CASES = [
    # seed, B, H, Hkv, Sq, Skv, d, dv, causal, kv_lens, masked
    (111, 1, 2, 2, 50, 50, 64, 16, 1, None, False),
    (112, 2, 4, 2, 33, 100, 16, 128, 1, [100, 41], False),
    (113, 1, 3, 1, 1, 300, 40, 100, 0, [250], False),
    (114, 2, 2, 2, 70, 90, 128, 7, 0, [90, 20], True),
    (115, 1, 2, 2, 65, 65, 3, 33, 1, None, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_value_width_matches_oracle(case):
    seed, B, H, Hkv, Sq, Skv, d, dv, causal, lens, masked = case
    _say(f"value width s{seed}: d {d} d_v {dv}")
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "f32", lens, dv=dv, Hkv=Hkv)
    mask = W.random_mask(seed, (B, 1, Sq, Skv), 0.6) if masked else None
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                     mask=None if mask is None else W.mask_to_torch(mask))
    assert got.shape == (B, H, Sq, dv)
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, clamped,
                           mask=mask)
    assert_matches(got, ref, F32_TOL, clamped, Skv, f"s{seed}")


BF16_CASES = [
    # seed, B, H, Hkv, Sq, Skv, d, dv, causal, kv_lens, extra
    (121, 2, 4, 2, 300, 300, 128, 64, 1, [300, 111], None),
    (122, 1, 4, 4, 515, 515, 64, 128, 1, None, None),
    (123, 1, 8, 8, 300, 6000, 64, 128, 1, None, None),        # key-range splits
    (124, 1, 8, 2, 200, 5000, 128, 64, 1, None, None),
    (125, 3, 4, 4, 1, 3000, 128, 64, 0, [3000, 17, 0], None),  # decode
    (126, 2, 32, 1, 1, 4100, 64, 128, 0, [4100, 900], None),  # decode, MQA
    (127, 2, 4, 2, 130, 260, 64, 128, 1, [260, 100], "mask"),
    (128, 2, 4, 4, 1, 2000, 128, 64, 0, [2000, 500], "mask"),
    (129, 2, 4, 2, 200, 200, 128, 64, 1, [200, 60], "bias"),
    (130, 2, 8, 2, 1, 1500, 64, 128, 0, [1500, 70], "bias"),
    # unsplit grids of 256-row blocks: with d = 64, d_v = 128 the outputs are
    # stored without the LDS staging, with d = 128, d_v = 64 the Q fragments
    # are loaded without it (the per-wave regions do not fit)
    (131, 3, 44, 4, 512, 512, 64, 128, 1, [512, 300, 17], None),
    (132, 3, 44, 4, 512, 512, 128, 64, 1, [512, 300, 17], None),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: f"s{c[0]}")
def test_bf16_value_width_matches_oracle(case):
    seed, B, H, Hkv, Sq, Skv, d, dv, causal, lens, extra = case
    _say(f"bf16 value width s{seed}: d {d} d_v {dv} {extra}")
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens, dv=dv, Hkv=Hkv)
    mask = W.random_mask(seed, (B, 1, Sq, Skv), 0.6) if extra == "mask" else None
    bias = W.random_bias(seed, (1, H, Sq, Skv), "bf16", hide=0.1) if extra == "bias" else None
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                     mask=None if mask is None else W.mask_to_torch(mask),
                     bias=None if bias is None else W.bias_to_torch(bias))
    assert got.shape == (B, H, Sq, dv)
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, clamped,
                           mask=mask, bias=bias)
    assert_matches(got, ref, BF16_TOL, clamped, Skv, f"s{seed}")


def test_bf16_rejects_other_value_widths():
    for dv in (32, 96):
        prob = W.random_problem(116, 1, 2, 8, 8, 64, "bf16", dv=dv)
        with pytest.raises(attn.AttnError) as e:
            gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
        assert e.value.status == attn.E_UNSUPPORTED
