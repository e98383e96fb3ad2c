"""GPU kernels against the CPU oracle on the same seeded bits (MI355X).

Small and ragged problems are compared element by element; the workloads at
full size run in the same launch configuration the benchmark times and are
compared on sampled (batch, head) slices, which the oracle computes on its
own (heads and batch items are independent).
"""
import math

import numpy as np
import pytest

import golden_io
import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, check_workload_full, check_problem, gpu_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- fp32 path
def test_tiny_f32_workload():
    w = W.WORKLOADS["tiny_f32"]
    x = W.make_inputs(w)
    _say("tiny_f32", w)
    got, _ = gpu_run(x["q"], x["k"], x["v"], x["scale"], w.causal)
    ref = oracle.attention(x["q"], x["k"], x["v"], x["scale"], w.causal)
    assert_matches(got, ref, F32_TOL, what="tiny_f32")


@pytest.mark.parametrize("name", ["p2_causal_3tok_d2.txt", "p3_unmasked_3tok_dk4_dv2.txt"])
def test_worked_examples_zero_padded(name):
    """The pages' two worked examples through the fp32 kernel: features
    zero-padded to 16 (zero features add nothing to a dot product, zero value
    columns give zero outputs), with the page's own scale."""
    g = golden_io.load(name)
    T = g["q"].shape[0]
    q = np.zeros((1, 1, T, 16), np.float32)
    k = np.zeros((1, 1, T, 16), np.float32)
    v = np.zeros((1, 1, T, 16), np.float32)
    q[0, 0, :, :g["q"].shape[1]] = g["q"]
    k[0, 0, :, :g["k"].shape[1]] = g["k"]
    v[0, 0, :, :g["v"].shape[1]] = g["v"]
    got, _ = gpu_run(q, k, v, float(np.float32(g["scale"])), g["causal"])
    ref = oracle.attention(q, k, v, float(np.float32(g["scale"])), g["causal"])
    assert_matches(got, ref, F32_TOL, what=name)
    oexp, otol = g["out"]
    dv = oexp.shape[1]
    assert np.all(np.abs(got[0, 0, :, :dv] - oexp) <= otol)
    assert np.all(got[0, 0, :, dv:] == 0.0)


F32_CASES = [
    # seed, B, H, Sq, Skv, d, causal, kv_lens
    (1, 1, 1, 64, 64, 16, 1, None),
    (2, 2, 3, 77, 77, 5, 1, None),
    (3, 2, 2, 130, 130, 33, 1, [130, 61]),
    (4, 1, 2, 100, 100, 64, 0, [57]),
    (5, 2, 1, 40, 129, 128, 1, [129, 80]),
    (6, 3, 2, 1, 300, 100, 0, [300, 1, 0]),
    (7, 1, 1, 1, 1, 1, 1, None),
    (8, 2, 2, 70, 70, 128, 1, [70, 0]),
    (9, 1, 3, 65, 65, 64, 1, [200]),          # length above capacity: clamped
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"s{c[0]}")
def test_f32_shapes(case):
    seed, B, H, Sq, Skv, d, causal, lens = case
    _say("f32 case", case)
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "f32", lens)
    check_problem(prob, causal, F32_TOL, f"f32 {case}")


# --------------------------------------------------------- bf16 prefill path
PREFILL_CASES = [
    (11, 1, 1, 64, 64, 128, 1, None),
    (12, 2, 3, 300, 300, 128, 1, None),
    (13, 1, 2, 200, 200, 64, 1, [137]),
    (14, 2, 2, 129, 129, 64, 1, [129, 3]),
    (15, 1, 2, 190, 190, 128, 0, None),
    (16, 2, 1, 257, 257, 128, 0, [250, 100]),
    (17, 1, 2, 70, 333, 128, 1, [300]),        # fewer queries than keys
    (18, 2, 2, 2, 515, 64, 1, [515, 40]),
    (19, 3, 1, 384, 384, 128, 1, [384, 1, 0]),
    (20, 1, 1, 2, 2, 128, 1, None),
    (21, 1, 4, 96, 96, 64, 0, None),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"s{c[0]}")
def test_bf16_prefill_shapes(case):
    seed, B, H, Sq, Skv, d, causal, lens = case
    _say("prefill case", case)
    assert attn.kernel_for(Sq, Skv, d, attn.BF16) == "prefill_bf16_mfma"
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens)
    check_problem(prob, causal, BF16_TOL, f"prefill {case}")


def _straddle(B, S, d, masked, rows):
    """Smallest H for which H and H + 1 heads of this shape take blocks of
    rows[0] and rows[1] query rows (unsplit)."""
    for H in range(1, 200):
        a = attn.prefill_plan(B, H, S, S, d, masked=masked)
        c = attn.prefill_plan(B, H + 1, S, S, d, masked=masked)
        if a[0] == c[0] == 1 and (a[1], c[1]) == rows:
            return H
    raise AssertionError(f"no head count switches {rows} at B={B} S={S}")


@pytest.mark.parametrize("rows", [(64, 128), (128, 256)])
@pytest.mark.parametrize("mask_kind", [None, "padding", "per_query"])
def test_block_height_does_not_change_rows(mask_kind, rows):
    """Small unsplit grids run blocks of 64 or 128 query rows, larger ones
    blocks of 256.  For each switch, H heads of 1000 rows take the smaller
    blocks and H + 1 heads the larger ones (H found from the launch plan).
    Both match the oracle, and the first H heads of the larger problem are
    bit-identical to the smaller one when both split their blocks' keys the
    same way: a row's result does not depend on the block height."""
    import torch
    B, S, d = 2, 1000, 128
    lens = [1000, 777]
    H = _straddle(B, S, d, mask_kind is not None, rows)
    prob = W.random_problem(91, B, H + 1, S, S, d, "bf16", lens)
    mask = None
    if mask_kind == "padding":
        mask = W.key_padding_mask([0, 64], lens, S)
    elif mask_kind == "per_query":
        mask = W.random_mask(92, (B, 1, S, S), 0.7)
    tm = None if mask is None else W.mask_to_torch(mask)
    plans = {h: attn.prefill_plan(B, h, S, S, d, masked=mask is not None) for h in (H, H + 1)}
    _say(f"block heights {rows}, mask {mask_kind}, H {H}: plans", plans)
    runs = {}
    for h in (H, H + 1):
        q, k, v = (np.ascontiguousarray(prob[x][:, :h]) for x in ("q", "k", "v"))
        got, out = gpu_run(q, k, v, prob["scale"], 1, lens, mask=tm)
        ref = oracle.attention(q, k, v, prob["scale"], 1, lens, mask=mask)
        assert_matches(got, ref, BF16_TOL, lens, S, f"H{h} mask {mask_kind}")
        runs[h] = out
    if plans[H][2] == plans[H + 1][2]:
        assert torch.equal(runs[H + 1][:, :H], runs[H]), "block height changed the rows"


# Small unmasked grids whose blocks split their keys between two wave sets
KEY_GROUP_CASES = [
    # seed, B, H, Sq, Skv, d, dv, causal, kv_lens
    (51, 1, 4, 1000, 1000, 64, 64, 1, None),
    (52, 1, 4, 777, 777, 128, 128, 1, [700]),
    (53, 2, 2, 513, 513, 64, 128, 0, [513, 200]),
    (54, 1, 2, 300, 1100, 128, 64, 1, None),     # fewer queries than keys
    (55, 1, 1, 576, 576, 64, 64, 1, None),       # an odd number of key tiles
    (56, 1, 1, 2, 600, 64, 64, 1, None),         # two queries, ten key tiles
    (57, 3, 2, 640, 640, 128, 128, 1, [640, 0, 65]),
    (58, 4, 12, 512, 512, 64, 64, 1, None),      # the mha768 shape
    (59, 1, 24, 2048, 2048, 128, 128, 1, None),  # 128-row blocks, two rounds of them
]
KEY_GROUP_KV_HEADS = {59: 6}  # grouped K/V heads for these seeds


@pytest.mark.parametrize("seed,Hkv", [(52, 2), (58, 3)])
def test_key_group_prefill_grouped_heads(seed, Hkv):
    """Key groups with grouped K/V heads equal the same call on K/V expanded
    to one head per query head, bit for bit (same plan, same bits read)."""
    case = next(c for c in KEY_GROUP_CASES if c[0] == seed)
    _, B, H, Sq, Skv, d, dv, causal, lens = case
    assert attn.prefill_plan(B, H, Sq, Skv, d, dv, H_kv=Hkv)[2] == 2
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens, dv=dv, Hkv=Hkv)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens)
    g = H // Hkv
    k = np.repeat(prob["k"], g, axis=1)
    v = np.repeat(prob["v"], g, axis=1)
    exp, _ = gpu_run(prob["q"], k, v, prob["scale"], causal, lens)
    assert np.array_equal(got, exp)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens)
    assert_matches(got, ref, BF16_TOL, lens, Skv, f"grouped key groups s{seed}")


@pytest.mark.parametrize("case", KEY_GROUP_CASES, ids=lambda c: f"s{c[0]}")
def test_key_group_prefill(case):
    """The plan splits these blocks' keys between two wave sets (tiles of each
    parity, two online softmaxes merged at the end); every element matches the
    oracle and padded rows are zero."""
    seed, B, H, Sq, Skv, d, dv, causal, lens = case
    plan = attn.prefill_plan(B, H, Sq, Skv, d, dv)
    _say("key-group case", case, "plan", plan)
    assert plan[0] == 1 and plan[2] == 2, plan
    Hkv = KEY_GROUP_KV_HEADS.get(seed, H)
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens, dv=dv, Hkv=Hkv)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens)
    assert_matches(got, ref, BF16_TOL, lens, Skv, f"key groups {case}")


# ---------------------------------------------------------- bf16 decode path
DECODE_CASES = [
    (31, 1, 1, 1, 1, 128, 0, None),
    (32, 3, 4, 1, 1000, 128, 0, [1, 513, 1000]),
    (33, 2, 3, 1, 700, 64, 0, [700, 65]),
    (34, 4, 2, 1, 2048, 128, 1, [0, 2048, 5000, 777]),
    (35, 1, 8, 1, 4100, 128, 0, None),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"s{c[0]}")
def test_bf16_decode_shapes(case):
    seed, B, H, Sq, Skv, d, causal, lens = case
    _say("decode case", case)
    assert attn.kernel_for(Sq, Skv, d, attn.BF16) == "decode_bf16_stream"
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens)
    check_problem(prob, causal, BF16_TOL, f"decode {case}")


# ------------------------------------------------- workloads at full size
def test_workload_mha768_full():
    check_workload_full(W.WORKLOADS["mha768_bf16"], say=print)


def test_workload_prefill4096_full():
    """Every head of the 4096-token causal prefill against the oracle."""
    check_workload_full(W.WORKLOADS["prefill4096_bf16"], say=print)


def test_workload_padded2048_full():
    """Every (b, h) of the padded batch (lengths U[256, 2048])."""
    check_workload_full(W.WORKLOADS["padded2048_bf16"], say=print)


def test_workload_decode8192_full():
    """Every (b, h) of the 64-sequence decode (lengths U[512, 8192])."""
    check_workload_full(W.WORKLOADS["decode8192_bf16"], say=print)


# ------------------------------------------- chunked prefill (1 < Sq < Skv)
def test_chunked_prefill_matches_full_prefill():
    """Cached vs uncached at scale: the last c rows of a causal prefill over S
    tokens equal a prefill of those c queries against the full S-key cache
    (bottom-right alignment).  The short chunk runs with its key range split
    over several blocks and merged, the full prefill without, so they agree
    to rounding; both are checked against the oracle on sampled heads."""
    import torch
    B, H, S, d = 1, 32, 2048, 128
    w = W.Workload("chunk_check", B, H, S, S, d, "bf16", True, 77)
    x = W.device_inputs(w)
    full = attn.fwd(x["q"], x["k"], x["v"], causal=True, scale=x["scale"])
    for c in (512, 100, 2):
        _say("chunked prefill, chunk", c, "plan workspace",
             attn.workspace_bytes(B, H, c, S, d, attn.BF16))
        qc = x["q"][:, :, S - c:].contiguous()
        part = attn.fwd(qc, x["k"], x["v"], causal=True, scale=x["scale"])
        torch.cuda.synchronize()
        got, ref = W.from_torch(part), W.from_torch(full[:, :, S - c:])
        assert np.max(np.abs(got - ref)) <= BF16_TOL, c
        sub = W.make_inputs(w, pairs=[(0, 0), (0, 21)])
        oref = oracle.attention(sub["q"][:, :, S - c:], sub["k"], sub["v"], sub["scale"], True)
        assert_matches(got[0, [0, 21]][:, None], oref, BF16_TOL, what=f"chunk {c}")


CHUNK_CASES = [
    # seed, B, H, Sq, Skv, d, causal, kv_lens: few query tiles against long caches
    (61, 1, 4, 300, 3000, 128, 1, None),
    (62, 2, 2, 2, 5000, 64, 1, [5000, 2047]),
    (63, 1, 8, 64, 4096, 128, 0, None),
    (64, 3, 1, 257, 2600, 128, 1, [2600, 300, 0]),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"s{c[0]}")
def test_split_prefill_shapes(case):
    seed, B, H, Sq, Skv, d, causal, lens = case
    _say("split prefill case", case, "workspace", attn.workspace_bytes(B, H, Sq, Skv, d, attn.BF16))
    assert attn.workspace_bytes(B, H, Sq, Skv, d, attn.BF16) > 0
    prob = W.random_problem(seed, B, H, Sq, Skv, d, "bf16", lens)
    check_problem(prob, causal, BF16_TOL, f"split prefill {case}")
