"""Explicit allowed-masks on the GPU against the CPU oracle.

The mask (True = may attend) is ANDed with the causal and length rules
("Attention from Scratch", KubeDojo module 1.4.3, Part 3).  Every kernel
family -- bf16 prefill (with and without key-range splits), the decode
stream kernel over its visible-tile lists (one and several query heads per
K/V head), the fp32 kernel -- runs masks in every broadcast shape on ragged
sizes (Skv not a multiple of the tiles, nor of 4) and is compared element by
element with the oracle; rows with no allowed key must be exactly zero.  An
all-true mask must give the unmasked result bit for bit (decode: to
rounding), and a mask spelling out the causal rule must reproduce the causal
result.
"""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, assert_matches, check_workload_full, gpu_run, key_groups

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


CASES = [
    # seed, dtype, B, H, Hkv, Sq, Skv, d, causal, kv_lens, mask shape (None = full), density
    (71, "bf16", 2, 4, 4, 300, 300, 128, 1, [300, 170], "b1qk", 0.7),
    (72, "bf16", 1, 2, 2, 129, 262, 64, 0, None, "1hqk", 0.5),
    (73, "bf16", 2, 4, 2, 256, 512, 128, 1, None, "bh1k", 0.8),
    (74, "bf16", 1, 2, 2, 200, 2602, 128, 1, [2602], "11qk", 0.3),   # key-range splits
    (75, "bf16", 2, 4, 4, 65, 131, 64, 0, [131, 40], "bhqk", 0.05),  # many empty rows
    (76, "bf16", 3, 4, 4, 1, 700, 128, 0, [700, 333, 0], "bh1k", 0.5),  # decode, one head per K/V head
    (77, "bf16", 2, 8, 4, 1, 1031, 64, 0, [1031, 500], "b11k", 0.6),  # decode, 2 heads per K/V head
    (78, "bf16", 2, 16, 2, 1, 1100, 128, 0, [1100, 900], "bh1k", 0.4),  # decode, 8 heads per K/V head
    (79, "bf16", 1, 32, 1, 1, 2049, 128, 0, None, "b11k", 0.02),
    (80, "f32", 2, 3, 3, 70, 90, 40, 1, [90, 50], "bhqk", 0.6),
    (81, "f32", 1, 4, 2, 1, 150, 128, 0, None, "1h1k", 0.5),
    # per-head planes (no key-tile lists) on whole 64-key tiles, 256-row
    # blocks: the mask words read by the block as 16-byte chunks
    (82, "bf16", 3, 48, 8, 512, 512, 128, 1, [512, 300, 17], "bhqk", 0.6),
]

_SHAPES = {"bhqk": "BHQK", "b1qk": "B1QK", "1hqk": "1HQK", "bh1k": "BH1K", "11qk": "11QK",
           "b11k": "B11K", "1h1k": "1H1K"}


def _mask_shape(code, B, H, Sq, Skv):
    dims = {"B": B, "H": H, "Q": Sq, "K": Skv, "1": 1}
    return tuple(dims[c] for c in _SHAPES[code])


def _run_case(case, mask):
    seed, dt, B, H, Hkv, Sq, Skv, d, causal, lens = case[:10]
    prob = W.random_problem(seed, B, H, Sq, Skv, d, dt, lens, Hkv=Hkv)
    q, k, v = prob["q"], prob["k"], prob["v"]
    got, _ = gpu_run(q, k, v, prob["scale"], causal, lens,
                     mask=None if mask is None else W.mask_to_torch(mask))
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    return got, prob, clamped


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_mask_matches_oracle(case):
    seed, dt, B, H, Hkv, Sq, Skv, d, causal, lens, shape, density = case
    _say(f"mask case s{seed}: {dt} B{B} H{H}/{Hkv} Sq{Sq} Skv{Skv} d{d} causal{causal} {shape}")
    mask = W.random_mask(seed, _mask_shape(shape, B, H, Sq, Skv), density)
    if shape == "bhqk" and Sq > 3:
        mask[0, 0, 3, :] = False  # one row with no allowed key
    got, prob, clamped = _run_case(case, mask)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, clamped,
                           mask=mask)
    tol = F32_TOL if dt == "f32" else BF16_TOL
    assert_matches(got, ref, tol, clamped, Skv, f"s{seed}")
    # rows the oracle gives no visible key are exactly zero on the GPU too
    empty = np.all(ref == 0.0, axis=-1)
    assert np.all(got[empty] == 0.0), f"s{seed}: rows without an allowed key are not zero"
    if shape == "bhqk" and Sq > 3:
        assert np.all(got[0, 0, 3] == 0.0)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}")
def test_all_true_mask_is_bitwise_unmasked(case):
    """Bit for bit, except bf16 decode (the masked stream kernel can hold a
    different number of resident waves than the unmasked one, d = 64, and so
    cut its shares of the keys elsewhere) and small unmasked prefills that
    split each block's keys between two wave sets; those agree to rounding."""
    seed, dt, B, H, Hkv, Sq, Skv, d, causal, lens = case[:10]
    _say(f"all-true mask s{seed}")
    ones = np.ones((1, 1, 1, Skv), dtype=bool)
    with_mask, _, _ = _run_case(case, ones)
    without, _, _ = _run_case(case, None)
    regrouped = key_groups(B, H, Sq, Skv, d, dtype=dt) != key_groups(B, H, Sq, Skv, d, dtype=dt,
                                                                       masked=True)
    if (dt == "bf16" and Sq == 1) or regrouped:
        clamped = None if lens is None else np.clip(lens, 0, Skv)
        assert_matches(with_mask, without, BF16_TOL, clamped, Skv, f"s{seed} masked vs stream")
    else:
        assert np.array_equal(with_mask, without), f"s{seed}: all-true mask changed the result"


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_causal_rule_as_mask(dt, d):
    """A [1,1,S,S] lower-triangular mask with causal off gives the causal result
    (equal values; the masked run also visits the tiles past the diagonal)."""
    import torch
    B, H, S = 2, 4, 333
    _say(f"causal-as-mask {dt} d{d}")
    prob = W.random_problem(90 + d, B, H, S, S, d, dt)
    tri = np.tril(np.ones((S, S), dtype=bool))[None, None]
    a, ta = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    b, tb = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, mask=W.mask_to_torch(tri))
    assert torch.equal(ta, tb), f"max diff {np.abs(a - b).max()}"


def _edge_mask(S):
    """Row i sees key 100 only, except row 255, which sees only key 63 (the
    last byte of the last row of query tile 0 in key tile 0), and row 511,
    which sees only key S - 1 (query tile 1's ragged last key tile): each of
    those two (query tile, key tile) blocks is visible through one byte."""
    m = np.zeros((S, S), dtype=bool)
    m[:, 100] = True
    m[255, 100] = False
    m[255, 63] = True
    m[511, 100] = False
    m[511, S - 1] = True
    return m[None, None]


STRUCTURED = [
    # name, B, H, S, d, causal, kv_lens, mask builder
    ("left padding", 2, 4, 1000, 128, 1, [1000, 700],
     lambda S: W.key_padding_mask([300, 130], [S, S], S)),
    ("documents", 1, 4, 1000, 128, 1, None, lambda S: W.document_mask([200, 577, 223])),
    ("documents d64", 1, 2, 777, 64, 0, None, lambda S: W.document_mask([64, 1, 300, 412])),
    ("sliding window", 1, 4, 1200, 128, 1, None, lambda S: W.window_mask(S, 130)),
    ("window split", 1, 2, 4500, 128, 0, None, lambda S: W.window_mask(S, 70)),
    ("tile edges only", 1, 2, 602, 128, 0, None, _edge_mask),
    # keys a multiple of 64 and 16-byte rows: the pre-pass reads 16 keys per load
    ("documents, whole key tiles", 1, 4, 1024, 128, 1, None,
     lambda S: W.document_mask([200, 577, 247])),
    ("tile edges only, whole key tiles", 1, 2, 640, 128, 0, None, _edge_mask),
    ("sliding window, whole key tiles", 1, 2, 1024, 64, 1, None, lambda S: W.window_mask(S, 100)),
]


@pytest.mark.parametrize("case", STRUCTURED, ids=lambda c: c[0].replace(" ", "_"))
def test_structured_masks_skip_hidden_tiles(case):
    """Masks that hide whole tiles from whole waves (those waves skip them)."""
    name, B, H, S, d, causal, lens, build = case
    _say(f"structured mask {name}: B{B} H{H} S{S} d{d} causal{causal}")
    prob = W.random_problem(sum(map(ord, name)), B, H, S, S, d, "bf16", lens)
    mask = build(S)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                     mask=W.mask_to_torch(mask))
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                           mask=mask)
    assert_matches(got, ref, BF16_TOL, lens, S, name)
    assert np.all(got[np.all(ref == 0.0, axis=-1)] == 0.0)


def _hole_mask(Sq, Skv, holes):
    m = np.ones((1, 1, Sq, Skv), dtype=bool)
    for i, j in holes:
        m[0, 0, i, j] = False
    return m


# name, B, H, Sq, Skv, d, causal, kv_lens, mask builder, equal to the unmasked run
WHOLE_TILES = [
    ("all-true plane", 2, 4, 700, 700, 128, 1, [700, 555],
     lambda B, Sq, Skv: np.ones((1, 1, Sq, Skv), dtype=bool), True),
    ("causal rule given with the rule", 2, 2, 600, 600, 64, 1, [600, 401],
     lambda B, Sq, Skv: np.tril(np.ones((Sq, Skv), dtype=bool))[None, None], True),
    ("zeros only above the diagonal", 1, 2, 300, 900, 128, 1, None,
     lambda B, Sq, Skv: _hole_mask(Sq, Skv, [(0, 601), (0, 899), (255, 856)]), True),
    ("one hidden byte per tile", 1, 2, 520, 520, 64, 0, None,
     lambda B, Sq, Skv: _hole_mask(Sq, Skv, [(0, 0), (255, 63), (256, 64), (519, 519), (300, 450)]),
     False),
    ("one hidden byte below the diagonal", 2, 2, 400, 400, 128, 1, [400, 390],
     lambda B, Sq, Skv: _hole_mask(Sq, Skv, [(399, 5), (256, 256)]), False),
    ("tile-aligned padding with splits", 2, 2, 200, 2602, 128, 1, [2602, 2000],
     lambda B, Sq, Skv: W.key_padding_mask([320, 130], [Skv, Skv], Skv), False),
    ("per-item padding, ragged", 3, 2, 333, 1030, 64, 0, [1030, 1000, 700],
     lambda B, Sq, Skv: W.key_padding_mask([0, 64, 192], [1030, 1030, 641], Skv), False),
    # whole key tiles and 16-byte rows (the pre-pass's 16-key loads)
    ("one hidden byte per tile, whole key tiles", 1, 2, 512, 512, 64, 0, None,
     lambda B, Sq, Skv: _hole_mask(Sq, Skv, [(0, 0), (255, 63), (256, 64), (511, 511), (300, 450)]),
     False),
    ("causal rule given with the rule, whole key tiles", 2, 2, 640, 640, 64, 1, [640, 401],
     lambda B, Sq, Skv: np.tril(np.ones((Sq, Skv), dtype=bool))[None, None], True),
    ("zeros only above the diagonal, whole key tiles", 1, 2, 300, 1024, 128, 1, None,
     lambda B, Sq, Skv: _hole_mask(Sq, Skv, [(0, 725), (0, 1023), (255, 980)]), True),
    # one-row masks past 64 key tiles take the pre-pass instead of the blocks' own marks
    ("long all-true row", 1, 2, 256, 5000, 64, 1, None,
     lambda B, Sq, Skv: np.ones((1, 1, 1, Skv), dtype=bool), True),
    ("long padding rows with splits", 2, 2, 300, 6000, 128, 1, [6000, 5000],
     lambda B, Sq, Skv: W.key_padding_mask([640, 100], [Skv, Skv], Skv), False),
]


@pytest.mark.parametrize("case", WHOLE_TILES, ids=lambda c: c[0].replace(" ", "_"))
def test_tiles_the_mask_opens_whole(case):
    """Blocks whose listed key tiles are consecutive and each opened whole by
    the mask run the unmasked loop; a single hidden byte, or a tile the mask
    cuts, sends the block back to the per-element path.  Bytes the causal
    rule hides anyway do not cut a tile."""
    name, B, H, Sq, Skv, d, causal, lens, build, same = case
    _say(f"whole-tile mask {name}: B{B} H{H} Sq{Sq} Skv{Skv} d{d} causal{causal}")
    prob = W.random_problem(sum(map(ord, name)), B, H, Sq, Skv, d, "bf16", lens)
    mask = build(B, Sq, Skv)
    got, tgot = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                        mask=W.mask_to_torch(mask))
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens,
                           mask=mask)
    assert_matches(got, ref, BF16_TOL, lens, Skv, name)
    if same:
        import torch
        plain_np, plain = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], causal, lens)
        if key_groups(B, H, Sq, Skv, d) == key_groups(B, H, Sq, Skv, d, masked=True):
            assert torch.equal(tgot, plain), f"{name}: differs from the unmasked run"
        else:  # the unmasked run splits its blocks' keys: equal to rounding
            assert_matches(got, plain_np, BF16_TOL, lens, Skv, f"{name} vs unmasked")


def test_whole_tile_mask_with_bias():
    """The general-logit kernel with an all-true mask equals the bias alone."""
    import torch
    Sq, Skv = 300, 700
    prob = W.random_problem(97, 2, 4, Sq, Skv, 128, "bf16", [700, 650], Hkv=2)
    bias = W.random_bias(98, (2, 4, Sq, Skv), "bf16", hide=0.05)
    tq, tk, tv = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    tl = torch.as_tensor(np.asarray([700, 650], np.int32)).to("cuda")
    tb = W.bias_to_torch(bias)
    a = attn.fwd(tq, tk, tv, causal=True, kv_lens=tl, scale=prob["scale"], bias=tb)
    m = W.mask_to_torch(np.ones((2, 1, Sq, Skv), dtype=bool))
    b = attn.fwd(tq, tk, tv, causal=True, kv_lens=tl, scale=prob["scale"], bias=tb, mask=m)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_mask_layout_errors():
    import torch
    B, H, S, d = 1, 2, 90, 64
    prob = W.random_problem(95, B, H, S, S, d, "bf16")
    q, k, v = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    dense = torch.ones((B, 1, S, S), dtype=torch.bool, device="cuda")  # rows of 90 bytes
    with pytest.raises((ValueError, attn.AttnError)):
        attn.fwd(q, k, v, mask=dense)
    wrong = torch.ones((B, 1, S, S + 1), dtype=torch.bool, device="cuda")
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, mask=wrong)
    ok = W.mask_to_torch(np.ones((B, 1, S, S), dtype=bool))
    out = attn.fwd(q, k, v, mask=ok)
    ref = attn.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_mask_decode_split_fully_hidden():
    """Decode with long key ranges hidden (no tile listed there) and a
    sequence whose every key is hidden (no tile listed at all: output 0), at
    one and at 8 query heads per K/V head."""
    for H, Hkv in ((8, 8), (16, 2)):
        B, Skv, d = 2, 3000, 128
        _say(f"decode hidden splits H{H}/{Hkv}")
        prob = W.random_problem(96 + H, B, H, 1, Skv, d, "bf16", Hkv=Hkv)
        starts, ends = [1700, 0], [2999, 0]
        mask = W.key_padding_mask(starts, ends, Skv)
        got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0,
                         mask=W.mask_to_torch(mask))
        ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0, mask=mask)
        assert_matches(got, ref, BF16_TOL, what=f"H{H}/{Hkv}")
        assert np.all(got[1] == 0.0)


def test_prefill4096_random_mask_full():
    """The 4096-token causal prefill in its benchmark launch configuration,
    with a random [1,1,S,S] mask (every tile cut), every head vs the oracle."""
    w = W.WORKLOADS["prefill4096_bf16"]
    check_workload_full(w, W.random_mask(97, (1, 1, w.Sq, w.Skv), 0.5), say=print)


def test_decode8192_key_padding_full():
    w = W.WORKLOADS["gqa_decode8192_bf16"]
    rng = np.random.default_rng(98)
    starts = rng.integers(0, 400, size=w.B)
    check_workload_full(w, W.key_padding_mask(starts, np.full(w.B, w.Skv), w.Skv), say=print)


def test_decode8192_random_head_mask_full():
    """Multi-head decode over the full workload with a per-head random mask:
    wave shares of listed tiles run past 128 entries, so the tile lists roll
    over in chunks of 64."""
    w = W.WORKLOADS["decode8192_bf16"]
    check_workload_full(w, W.random_mask(99, (w.B, w.H, 1, w.Skv), 0.5), say=print)


def test_decode_sparse_visible_windows():
    """Long caches where a few windows far apart are visible (listed tiles
    far apart), per head and shared, one sequence with nothing visible."""
    B, H, Hkv, Skv, d = 3, 8, 2, 20000, 128
    for shared in (False, True):
        _say(f"sparse windows shared={shared}")
        prob = W.random_problem(131 + shared, B, H, 1, Skv, d, "bf16", [20000, 17001, 9000],
                                Hkv=Hkv)
        mask = np.zeros((B, 1 if shared else H, 1, Skv), dtype=bool)
        for b in range(B - 1):
            for hh in range(mask.shape[1]):
                for lo in (37 + 101 * hh, 5000 + 7 * hh, 16990):
                    mask[b, hh, 0, lo:lo + 45] = True
        got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0,
                         [20000, 17001, 9000], mask=W.mask_to_torch(mask))
        ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0,
                               [20000, 17001, 9000], mask=mask)
        assert_matches(got, ref, BF16_TOL, what=f"sparse shared={shared}")
        assert np.all(got[B - 1] == 0.0)



def test_decode_mask_past_one_prepass_chunk():
    """A masked decode over more than 65536 keys: the visible-tile pre-pass
    flags tiles in LDS chunks of 2048 tiles, so its lists span two chunks."""
    B, H, Hkv, Skv, d = 2, 4, 2, 70000, 128
    lens = [70000, 66001]
    for shape in ((B, H, 1, Skv), (B, 1, 1, Skv)):
        _say(f"decode 70000 keys, mask {shape}")
        prob = W.random_problem(141 + len(shape), B, H, 1, Skv, d, "bf16", lens, Hkv=Hkv)
        mask = W.random_mask(141, shape, 0.02)
        mask[..., 65530:65560] = True  # keys both sides of the chunk edge
        got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens,
                         mask=W.mask_to_torch(mask))
        ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens,
                               mask=mask)
        assert_matches(got, ref, BF16_TOL, what=f"70000 keys {shape}")


def test_masked_decode_caller_workspace():
    """A masked decode with a caller workspace of workspace_bytes(masked=True)
    gives the bits of the library-owned one; one sized for the unmasked call
    (no room for the visible-tile lists) is refused."""
    import torch
    B, H, Hkv, Skv, d = 3, 8, 2, 3000, 128
    lens = [3000, 17, 2000]
    prob = W.random_problem(151, B, H, 1, Skv, d, "bf16", lens, Hkv=Hkv)
    q, k, v = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    tl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mask = W.mask_to_torch(W.random_mask(151, (B, H, 1, Skv), 0.3))
    ref = attn.fwd(q, k, v, causal=False, kv_lens=tl, mask=mask)
    need = attn.workspace_bytes(B, H, 1, Skv, d, attn.BF16, kv_heads=Hkv, masked=True)
    plain = attn.workspace_bytes(B, H, 1, Skv, d, attn.BF16, kv_heads=Hkv)
    assert need > plain
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = attn.fwd(q, k, v, causal=False, kv_lens=tl, mask=mask, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    with pytest.raises(attn.AttnError) as e:
        attn.fwd(q, k, v, causal=False, kv_lens=tl, mask=mask, workspace=ws[:plain])
    assert e.value.status == attn.E_WORKSPACE
    # the unmasked call runs in the smaller buffer
    out2 = attn.fwd(q, k, v, causal=False, kv_lens=tl, workspace=ws[:plain])
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16),
                       attn.fwd(q, k, v, causal=False, kv_lens=tl).view(torch.int16))
