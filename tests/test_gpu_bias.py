"""Additive bias and non-positive scales on the GPU (MI355X) against the oracle.

The bias is added to the scaled logits before the softmax ("Attention from
Scratch", KubeDojo module 1.4.3, Part 7: a float mask acts as an additive
bias); -inf hides a key exactly as a False mask byte does.  It has the
inputs' element type.  Every kernel family runs it: the fp32 kernel, and the
bf16 prefill and decode in their general instantiations, which also serve a
scale of zero or below."""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, check_workload_full

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(prob, causal, scale, bias_np=None, mask_np=None):
    import torch
    tq, tk, tv = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    lens = prob["kv_lens"]
    tl = None if lens is None else torch.as_tensor(np.asarray(lens, np.int32)).to("cuda")
    out = attn.fwd(tq, tk, tv, causal=bool(causal), kv_lens=tl, scale=scale,
                   bias=None if bias_np is None else W.bias_to_torch(bias_np),
                   mask=None if mask_np is None else W.mask_to_torch(mask_np))
    torch.cuda.synchronize()
    return W.from_torch(out)


def _check(prob, causal, scale, bias_np=None, mask_np=None, tol=BF16_TOL, what=""):
    got = _run(prob, causal, scale, bias_np, mask_np)
    Skv = prob["k"].shape[2]
    lens = prob["kv_lens"]
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], scale, causal, clamped,
                           mask=mask_np, bias=bias_np)
    return assert_matches(got, ref, tol, clamped, Skv, what)


# seed, B, H, H_kv, Sq, Skv, d, causal, lengths, bias shape kind, fraction hidden
CASES = [
    (1, 1, 2, 2, 200, 200, 128, 1, None, "full", 0.0),
    (2, 2, 4, 2, 515, 515, 128, 1, [515, 300], "heads", 0.1),
    (3, 2, 2, 1, 130, 700, 64, 1, [700, 129], "batch", 0.0),
    (4, 1, 3, 3, 2, 9, 128, 0, None, "rows", 0.2),
    (5, 3, 2, 2, 64, 64, 64, 0, [64, 1, 0], "full", 0.5),
    (6, 1, 8, 8, 300, 6000, 128, 1, None, "heads", 0.0),    # key-range splits
    (7, 2, 4, 4, 1, 3000, 128, 0, [3000, 1000], "heads", 0.3),   # decode
    (8, 3, 8, 2, 1, 900, 64, 0, [900, 31, 0], "batch", 0.0),    # decode, GQA
    (9, 1, 32, 1, 1, 4100, 128, 0, [4100], "heads", 0.1),     # decode, MQA
    # whole 64-key tiles: bias rows read by the block as 16-byte chunks, with
    # ragged lengths (dead rows in a sequence's first query tile), at block
    # heights 64 and 256
    (10, 2, 4, 2, 640, 640, 128, 1, [640, 333], "heads", 0.1),
    (11, 3, 48, 8, 512, 512, 128, 1, [512, 300, 17], "heads", 0.1),
]


def _bias_shape(kind, B, H, Sq, Skv):
    return {"full": (B, H, Sq, Skv), "heads": (1, H, Sq, Skv), "batch": (B, 1, Sq, Skv),
            "rows": (1, 1, 1, Skv)}[kind]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_bf16_bias(case):
    seed, B, H, Hkv, Sq, Skv, d, causal, lens, kind, hide = case
    _say("bias case", case)
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens, Hkv=Hkv)
    bias = W.random_bias(seed, _bias_shape(kind, B, H, Sq, Skv), "bf16", hide=hide)
    _check(prob, causal, prob["scale"], bias, what=f"bias {case}")


@pytest.mark.parametrize("case", CASES[:5], ids=lambda c: f"s{c[0]}")
def test_f32_bias(case):
    seed, B, H, Hkv, Sq, Skv, d, causal, lens, kind, hide = case
    _say("fp32 bias case", case)
    prob = W.random_problem(seed, B, H, Sq, Skv, min(d, 64), "f32", lens, Hkv=Hkv)
    bias = W.random_bias(seed, _bias_shape(kind, B, H, Sq, Skv), "f32", hide=hide)
    _check(prob, causal, prob["scale"], bias, tol=F32_TOL, what=f"fp32 bias {case}")


def test_bias_with_mask():
    """A bias and a boolean mask together (both ANDed/added with the rules)."""
    for Sq, Skv, d in ((300, 300, 128), (1, 2000, 128), (100, 130, 64)):
        _say("bias with mask", Sq, Skv, d)
        prob = W.random_problem(20 + Sq, 2, 4, Sq, Skv, d, "bf16", [Skv, Skv // 2], Hkv=2)
        bias = W.random_bias(21, (2, 4, Sq, Skv), "bf16", hide=0.05)
        mask = W.random_mask(22, (2, 1, Sq, Skv), 0.7)
        _check(prob, 1 if Sq > 1 else 0, prob["scale"], bias, mask, what=f"bias+mask {Sq}")


def test_neg_inf_bias_hides_every_key_of_a_row():
    """Rows whose bias hides every visible key are exactly zero."""
    for Sq, Skv in ((70, 70), (1, 500)):
        prob = W.random_problem(30, 1, 2, Sq, Skv, 128, "bf16")
        bias = W.random_bias(31, (1, 2, Sq, Skv), "bf16")
        bias[0, 1, 0, :] = W.bf16_bits(np.array([-np.inf], np.float32))[0]
        got = _run(prob, 1 if Sq > 1 else 0, prob["scale"], bias)
        assert np.all(got[0, 1, 0] == 0.0)
        _check(prob, 1 if Sq > 1 else 0, prob["scale"], bias, what="rows hidden")


@pytest.mark.parametrize("scale", [0.0, -0.0883883, -1.5])
def test_non_positive_scale(scale):
    """A scale of zero or below (any finite scale is a valid multiplier)."""
    for Sq, Skv, d, lens in ((257, 257, 128, [257, 100]), (1, 1500, 64, [1500, 3])):
        _say("scale", scale, Sq, Skv, d)
        prob = W.random_problem(40, 2, 2, Sq, Skv, d, "bf16", lens)
        _check(prob, 1 if Sq > 1 else 0, scale, what=f"scale {scale}")
        p32 = W.random_problem(41, 2, 2, Sq, Skv, 32, "f32", lens)
        _check(p32, 1 if Sq > 1 else 0, scale, tol=F32_TOL, what=f"fp32 scale {scale}")


def test_prefill4096_bias_full():
    """The 4096-token causal prefill with a [1,1,S,S] bias (a hidden tenth of
    the entries), every head against the oracle."""
    w = W.WORKLOADS["prefill4096_bf16"]
    check_workload_full(w, say=print, bias_np=W.random_bias(50, (1, 1, w.Sq, w.Skv), "bf16",
                                                            hide=0.1))


def test_decode8192_bias_full():
    """The 64-sequence decode with a per-head bias, every (b, h)."""
    w = W.WORKLOADS["decode8192_bf16"]
    check_workload_full(w, say=print, bias_np=W.random_bias(51, (w.B, w.H, 1, w.Skv), "bf16",
                                                            hide=0.05))
