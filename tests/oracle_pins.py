"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Every pin takes ``attn`` -- a callable with the signature of
``oracle.attention`` -- and raises AssertionError when it fails.  The same
pins run against the real oracle (all must pass) and against builds of the
oracle with a planted mistake (each build must fail at least one), so that a
plausible mistake anywhere in the oracle is shown to be caught.
"""
from __future__ import annotations

import math

import numpy as np

import golden_io
from workloads import bf16_bits, bf16_to_f32


def _rand(seed, *shape):
    return np.random.default_rng(np.random.SeedSequence([seed, 7])).standard_normal(shape)


def _fixture_case(attn, name):
    g = golden_io.load(name)
    q, k, v = (g[x][None, None] for x in ("q", "k", "v"))
    out, w = attn(q, k, v, g["scale"], g["causal"], weights=True)
    wexp, wtol = g["weights"]
    oexp, otol = g["out"]
    assert np.all(np.abs(w[0, 0] - wexp) <= wtol), f"{name}: weights {w[0, 0]} vs {wexp}"
    assert np.all(np.abs(out[0, 0] - oexp) <= otol), f"{name}: out {out[0, 0]} vs {oexp}"


def pin_p2_causal_example(attn):
    """"Attention from First Principles", section 4: the hand-worked causal
    example, and its remark that token 0 gets V[0] unchanged."""
    _fixture_case(attn, "p2_causal_3tok_d2.txt")
    g = golden_io.load("p2_causal_3tok_d2.txt")
    out = attn(g["q"][None, None], g["k"][None, None], g["v"][None, None], g["scale"], 1)
    assert np.array_equal(out[0, 0, 0], g["v"][0]), "row 0 must equal V[0] exactly"


def pin_p3_unmasked_example(attn):
    """KubeDojo "Attention from Scratch" (module 1.4.3), Part 2 worked example (d_v != d_k)."""
    _fixture_case(attn, "p3_unmasked_3tok_dk4_dv2.txt")


def _mixed_cases():
    # (B, H, Sq, Skv, d, causal, kv_lens)
    return [
        (2, 2, 5, 5, 3, 1, None),
        (2, 1, 6, 6, 4, 1, [6, 3]),
        (3, 2, 2, 7, 3, 1, [7, 4, 1]),
        (1, 2, 4, 7, 2, 0, None),
        (2, 1, 1, 9, 5, 0, [9, 2]),
        (2, 2, 7, 7, 2, 0, [5, 7]),
        (1, 1, 1, 1, 1, 1, None),
    ]


def _visible(Sq, Skv, causal, L):
    """Allowed-mask [Sq, Skv] and pad-row flags under the bottom-right reading."""
    n = min(Sq, L)
    allowed = np.zeros((Sq, Skv), dtype=bool)
    for i in range(n):
        p = L - n + i
        for j in range(L):
            allowed[i, j] = (not causal) or j <= p
    return allowed, np.arange(Sq) >= n


def pin_row_sums_and_forbidden_zero(attn):
    """Rows of weights sum to one over visible keys, and every forbidden entry
    (future key, pad key, pad query row) is exactly zero -- the invariants the
    "Attention from scratch" pages assert (Open LLM Engineering's readable model
    and KubeDojo Part 7: rows sum to one; weights for
    positions after the first are all zero in row 0; upper triangle zero)."""
    for ci, (B, H, Sq, Skv, d, causal, lens) in enumerate(_mixed_cases()):
        q, k, v = _rand(ci, B, H, Sq, d), _rand(ci + 50, B, H, Skv, d), _rand(ci + 90, B, H, Skv, d)
        out, w = attn(q, k, v, 1 / math.sqrt(d), causal, lens, weights=True)
        for b in range(B):
            L = Skv if lens is None else lens[b]
            allowed, pad = _visible(Sq, Skv, causal, L)
            for h in range(H):
                assert np.all(w[b, h][~allowed] == 0.0), f"case {ci}: forbidden weight nonzero"
                sums = w[b, h].sum(axis=-1)
                assert np.all(np.abs(sums[~pad] - 1.0) <= 1e-12), f"case {ci}: row sums {sums}"
                assert np.all(out[b, h][pad] == 0.0), f"case {ci}: pad row output nonzero"
                assert np.all(w[b, h][pad] == 0.0), f"case {ci}: pad row weights nonzero"


def pin_future_invariance(attn):
    """Under the causal mask, changing keys/values at positions >= t leaves
    every query row at a position < t bitwise unchanged."""
    B, H, S, d = 1, 2, 8, 4
    q, k, v = _rand(1, B, H, S, d), _rand(2, B, H, S, d), _rand(3, B, H, S, d)
    base = attn(q, k, v, 0.5, 1)
    for t in range(1, S):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, t:] = _rand(10 + t, B, H, S - t, d) * 3.0
        v2[:, :, t:] = _rand(40 + t, B, H, S - t, d) * 3.0
        out = attn(q, k2, v2, 0.5, 1)
        assert np.array_equal(out[:, :, :t], base[:, :, :t]), f"rows < {t} changed"
        assert not np.array_equal(out[:, :, t:], base[:, :, t:]), "later rows must see the change"


def pin_zero_query_uniform(attn):
    """With Q = 0 every visible key gets the same weight, so each output row is
    the plain mean of its visible value rows (the all-zero exercise on the
    Open LLM Engineering "Attention from scratch" exercises); np.mean is the
    independent reference."""
    B, H, S, d = 2, 1, 6, 3
    q = np.zeros((B, H, S, d))
    k, v = _rand(4, B, H, S, d), _rand(5, B, H, S, d)
    lens = [6, 4]
    out = attn(q, k, v, 0.7, 1, lens)
    for b in range(B):
        L = lens[b]
        for i in range(S):
            if i >= L:
                assert np.all(out[b, 0, i] == 0.0)
                continue
            ref = v[b, 0, : i + 1].mean(axis=0)
            assert np.allclose(out[b, 0, i], ref, rtol=0, atol=1e-12), (b, i)
    # decode: one query at the last valid position sees keys 0..L-1
    out = attn(q[:, :, :1], k, v, 0.7, 0, lens)
    for b in range(B):
        ref = v[b, 0, : lens[b]].mean(axis=0)
        assert np.allclose(out[b, 0, 0], ref, rtol=0, atol=1e-12)


def pin_convex_mixture(attn):
    """Each output is a convex mixture of the visible value rows, so every
    component lies between their minimum and maximum."""
    B, H, S, d = 1, 3, 9, 4
    q, k, v = _rand(6, B, H, S, d) * 3, _rand(7, B, H, S, d) * 3, _rand(8, B, H, S, d)
    out = attn(q, k, v, 0.5, 1)
    for h in range(H):
        for i in range(S):
            lo, hi = v[0, h, : i + 1].min(axis=0), v[0, h, : i + 1].max(axis=0)
            assert np.all(out[0, h, i] >= lo - 1e-12) and np.all(out[0, h, i] <= hi + 1e-12)


def pin_shift_invariance_large_logits(attn):
    """softmax is unchanged when one constant is added to every logit of a row.
    An extra feature with q_e = c and k_e = 1 adds scale*c to every logit; at
    c = 2e3 an implementation that does not subtract the row maximum
    overflows."""
    B, H, S, d = 1, 1, 6, 3
    q, k, v = _rand(9, B, H, S, d), _rand(10, B, H, S, d), _rand(11, B, H, S, d)
    base = attn(q, k, v, 0.5, 1)
    q2 = np.concatenate([q, np.full((B, H, S, 1), 2000.0)], axis=-1)
    k2 = np.concatenate([k, np.ones((B, H, S, 1))], axis=-1)
    out = attn(q2, k2, v, 0.5, 1)
    assert np.all(np.isfinite(out)), "large logits overflowed"
    assert np.allclose(out, base, rtol=0, atol=1e-9)


def pin_two_key_logistic(attn):
    """Two keys, no mask, d = 1: the weight of key 1 is the logistic function
    of the logit difference, sigma(scale*q*(k1 - k0)) (textbook identity)."""
    from scipy.special import expit
    rng = np.random.default_rng(12)
    for _ in range(20):
        q = rng.standard_normal((1, 1, 1, 1))
        k = rng.standard_normal((1, 1, 2, 1))
        v = np.array([[[[0.0], [1.0]]]])
        scale = float(rng.uniform(0.1, 2.0))
        out = attn(q, k, v, scale, 0)
        ref = expit(scale * q[0, 0, 0, 0] * (k[0, 0, 1, 0] - k[0, 0, 0, 0]))
        assert abs(out[0, 0, 0, 0] - ref) <= 1e-14, (out, ref)


def pin_matches_torch_sdpa(attn):
    """Agreement with an independent library routine: torch's CPU
    scaled_dot_product_attention in float64 (the comparison the KubeDojo
    page's test script makes), with the boolean allowed-mask built from the
    causal and padding rules."""
    import torch
    import torch.nn.functional as F
    for ci, (B, H, Sq, Skv, d, causal, lens) in enumerate(_mixed_cases()):
        q, k, v = _rand(ci, B, H, Sq, d), _rand(ci + 50, B, H, Skv, d), _rand(ci + 90, B, H, Skv, d)
        out = attn(q, k, v, 1 / math.sqrt(d), causal, lens)
        for b in range(B):
            L = Skv if lens is None else lens[b]
            allowed, pad = _visible(Sq, Skv, causal, L)
            rows = np.nonzero(~pad)[0]
            if len(rows) == 0:
                continue
            tq = torch.from_numpy(q[b][:, rows])
            ref = F.scaled_dot_product_attention(
                tq, torch.from_numpy(k[b]), torch.from_numpy(v[b]),
                attn_mask=torch.from_numpy(allowed[rows]), scale=1 / math.sqrt(d)).numpy()
            assert np.allclose(out[b][:, rows], ref, rtol=0, atol=1e-12), f"case {ci} b {b}"


def pin_decode_is_last_prefill_row(attn):
    """A single decode query against the cache equals the last row of causal
    prefill over the same keys (cached and uncached generation agree)."""
    B, H, S, d = 2, 2, 7, 3
    q, k, v = _rand(13, B, H, S, d), _rand(14, B, H, S, d), _rand(15, B, H, S, d)
    lens = [7, 5]
    full = attn(q, k, v, 0.6, 1, lens)
    for b in range(B):
        L = lens[b]
        qd = q[b:b + 1, :, L - 1:L]
        dec = attn(qd, k[b:b + 1], v[b:b + 1], 0.6, 0, [L])
        assert np.allclose(dec[0, :, 0], full[b, :, L - 1], rtol=0, atol=1e-13)
        dec1 = attn(qd, k[b:b + 1], v[b:b + 1], 0.6, 1, [L])
        assert np.array_equal(dec1, dec), "causal flag must not matter for one query"


def pin_key_permutation_equivariance(attn):
    """Without a mask, permuting keys together with their values leaves the
    output unchanged; permuting heads permutes outputs."""
    B, H, S, d = 1, 3, 6, 4
    q, k, v = _rand(16, B, H, 4, d), _rand(17, B, H, S, d), _rand(18, B, H, S, d)
    base = attn(q, k, v, 0.5, 0)
    perm = np.random.default_rng(3).permutation(S)
    out = attn(q, k[:, :, perm], v[:, :, perm], 0.5, 0)
    assert np.allclose(out, base, rtol=0, atol=1e-13)
    hp = [2, 0, 1]
    out = attn(q[:, hp], k[:, hp], v[:, hp], 0.5, 0)
    assert np.array_equal(out, base[:, hp])


def pin_low_precision_inputs_widen_exactly(attn):
    """bfloat16 bit patterns and float32 inputs are read as their exact values:
    results equal those of the same numbers passed as float64."""
    B, H, S, d = 1, 2, 5, 4
    x = [_rand(20 + i, B, H, S, d).astype(np.float32) for i in range(3)]
    ref32 = attn(*(a.astype(np.float64) for a in x), 0.5, 1)
    assert np.array_equal(attn(*x, 0.5, 1), ref32)
    bits = [bf16_bits(a) for a in x]
    ref16 = attn(*(bf16_to_f32(b).astype(np.float64) for b in bits), 0.5, 1)
    assert np.array_equal(attn(*bits, 0.5, 1), ref16)


def pin_length_clamp(attn):
    """Valid lengths are clamped to [0, Skv]: a length above capacity equals
    capacity, and a non-positive length gives an all-zero sequence."""
    B, H, S, d = 3, 1, 4, 2
    q, k, v = _rand(30, B, H, S, d), _rand(31, B, H, S, d), _rand(32, B, H, S, d)
    a = attn(q, k, v, 0.5, 1, [S + 5, 0, -3])
    b = attn(q, k, v, 0.5, 1, [S, 0, 0])
    assert np.array_equal(a, b)
    assert np.all(a[1:] == 0.0)


def pin_grouped_heads_match_expansion(attn):
    """Grouped key/value heads ("Scaled dot-product attention with masking",
    section "Grouped-query attention (GQA)"): the result equals plain
    multi-head attention after K and V are expanded along the head axis with
    repeat_interleave, here computed by torch's CPU scaled_dot_product_attention
    in float64 on the expanded tensors (an independent routine).  Covers MQA
    (one K/V head), GQA and MHA, causal with right padding, and B > 1."""
    import torch
    import torch.nn.functional as F
    B, H, Sq, Skv, d = 2, 4, 5, 7, 3
    lens = [7, 4]
    for ci, Hkv in enumerate((1, 2, 4)):
        q = _rand(60 + ci, B, H, Sq, d)
        k, v = _rand(70 + ci, B, Hkv, Skv, d), _rand(80 + ci, B, Hkv, Skv, d)
        out = attn(q, k, v, 0.7, 1, lens)
        ke = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
        ve = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
        for b in range(B):
            allowed, pad = _visible(Sq, Skv, 1, lens[b])
            rows = np.nonzero(~pad)[0]
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q[b][:, rows]), ke[b], ve[b],
                attn_mask=torch.from_numpy(allowed[rows]), scale=0.7).numpy()
            assert np.allclose(out[b][:, rows], ref, rtol=0, atol=1e-12), f"Hkv {Hkv} b {b}"
            assert np.all(out[b][:, pad] == 0.0)


def _random_mask(seed, shape, density=0.6):
    return np.random.default_rng(np.random.SeedSequence([seed, 11])).random(shape) < density


def pin_mask_of_the_rules_equals_the_rules(attn):
    """An allowed-mask that spells out the causal rule ("Self-Attention",
    section "Causal Masking", bottom-right aligned) with the causal flag off
    gives exactly the causal result, and an all-true mask exactly the
    unmasked one: the explicit mask and the built-in rules are one AND
    ("Attention from Scratch", KubeDojo module 1.4.3, Part 3)."""
    for ci, (B, H, Sq, Skv, d, causal, lens) in enumerate(_mixed_cases()):
        q, k, v = _rand(ci, B, H, Sq, d), _rand(ci + 50, B, H, Skv, d), _rand(ci + 90, B, H, Skv, d)
        ref = attn(q, k, v, 0.6, 1, lens)
        full = np.zeros((B, 1, Sq, Skv), dtype=bool)
        for b in range(B):
            L = Skv if lens is None else min(lens[b], Skv)
            allowed, _ = _visible(Sq, Skv, 1, L)
            full[b, 0] = allowed
        assert np.array_equal(attn(q, k, v, 0.6, 0, lens, mask=full), ref), f"case {ci}"
        assert np.array_equal(attn(q, k, v, 0.6, 1, lens, mask=full), ref), f"case {ci} both"
        ones = np.ones((1, 1, 1, Skv), dtype=np.uint8)
        assert np.array_equal(attn(q, k, v, 0.6, causal, lens, mask=ones),
                              attn(q, k, v, 0.6, causal, lens)), f"case {ci} all-true"


def pin_key_padding_mask_equals_lengths(attn):
    """A key-padding mask [B,1,1,Skv] (the padding mask of "Attention from
    Scratch", Part 3, broadcast over heads and queries) equals the valid
    lengths on every query row they both compute (rows i < L_b of a square
    problem, where the bottom-right offset is 0)."""
    B, H, S, d = 3, 2, 6, 3
    q, k, v = _rand(40, B, H, S, d), _rand(41, B, H, S, d), _rand(42, B, H, S, d)
    lens = [6, 4, 1]
    kp = (np.arange(S)[None, :] < np.array(lens)[:, None])[:, None, None, :]
    for causal in (0, 1):
        by_len = attn(q, k, v, 0.8, causal, lens)
        by_mask = attn(q, k, v, 0.8, causal, mask=kp)
        for b in range(B):
            assert np.array_equal(by_mask[b, :, :lens[b]], by_len[b, :, :lens[b]]), (causal, b)


def pin_mask_single_allowed_key(attn):
    """A row allowed exactly one key puts all its weight there: the output is
    that key's value row exactly (softmax over one logit is 1), and a row
    allowed no key is exactly zero."""
    B, H, Sq, Skv, d = 2, 2, 4, 6, 3
    q, k, v = _rand(43, B, H, Sq, d), _rand(44, B, H, Skv, d), _rand(45, B, H, Skv, d)
    pick = np.random.default_rng(5).integers(0, Skv, size=(B, H, Sq))
    m = np.zeros((B, H, Sq, Skv), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                m[b, h, i, pick[b, h, i]] = 7  # any nonzero byte allows
    m[1, 0, 2, :] = 0
    out, w = attn(q, k, v, 0.9, 0, mask=m, weights=True)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                if b == 1 and h == 0 and i == 2:
                    assert np.all(out[b, h, i] == 0.0) and np.all(w[b, h, i] == 0.0)
                    continue
                assert np.array_equal(out[b, h, i], v[b, h, pick[b, h, i]]), (b, h, i)
                assert w[b, h, i, pick[b, h, i]] == 1.0


def pin_mask_matches_torch_sdpa(attn):
    """Random allowed-masks in every broadcast shape, with the causal rule,
    valid lengths and grouped heads, against torch's CPU
    scaled_dot_product_attention in float64 given the AND of the mask and the
    rules (an independent routine).  Rows with no allowed key (where torch
    returns NaN) are exactly zero here, and every disallowed weight is 0."""
    import torch
    import torch.nn.functional as F
    B, H, Hkv, Sq, Skv, d = 2, 4, 2, 5, 7, 3
    lens = [7, 5]
    for ci, shape in enumerate([(B, H, Sq, Skv), (B, 1, Sq, Skv), (1, H, Sq, Skv),
                                (B, H, 1, Skv), (1, 1, Sq, Skv)]):
        m = _random_mask(ci, shape)
        causal = ci % 2
        q = _rand(100 + ci, B, H, Sq, d)
        k, v = _rand(110 + ci, B, Hkv, Skv, d), _rand(120 + ci, B, Hkv, Skv, d)
        out, w = attn(q, k, v, 0.7, causal, lens, mask=m, weights=True)
        mm = np.broadcast_to(m, (B, H, Sq, Skv))
        ke = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
        ve = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
        for b in range(B):
            rule, pad = _visible(Sq, Skv, causal, lens[b])
            for h in range(H):
                allowed = mm[b, h] & rule
                assert np.all(w[b, h][~allowed] == 0.0), (ci, b, h)
                rows = np.nonzero(allowed.any(axis=1))[0]
                empty = np.nonzero(~allowed.any(axis=1))[0]
                assert np.all(out[b, h, empty] == 0.0), (ci, b, h)
                if len(rows) == 0:
                    continue
                ref = F.scaled_dot_product_attention(
                    torch.from_numpy(q[b, h, rows]), ke[b, h], ve[b, h],
                    attn_mask=torch.from_numpy(np.ascontiguousarray(allowed[rows])),
                    scale=0.7).numpy()
                assert np.allclose(out[b, h, rows], ref, rtol=0, atol=1e-12), (ci, b, h)


def _bias_case(ci):
    B, H, Hkv, Sq, Skv, d = 2, 4, 2, 5, 7, 3
    q = _rand(200 + ci, B, H, Sq, d)
    k, v = _rand(210 + ci, B, Hkv, Skv, d), _rand(220 + ci, B, Hkv, Skv, d)
    return q, k, v, [7, 5]


def pin_zero_bias_is_no_bias(attn):
    """Adding a zero bias to every logit changes no bit of the output or the
    weights (causal, padded, grouped heads, with and without a mask)."""
    for ci in range(2):
        q, k, v, lens = _bias_case(ci)
        zero = np.zeros((1, 1, q.shape[2], k.shape[2]))
        m = _random_mask(300 + ci, (q.shape[0], 1, q.shape[2], k.shape[2])) if ci else None
        a, wa = attn(q, k, v, 0.6, 1, lens, mask=m, weights=True)
        b, wb = attn(q, k, v, 0.6, 1, lens, mask=m, bias=zero, weights=True)
        assert np.array_equal(a, b) and np.array_equal(wa, wb)


def pin_neg_inf_bias_is_the_boolean_mask(attn):
    """A bias of 0 where a boolean mask allows and -inf where it forbids is
    that mask ("Attention from Scratch", KubeDojo module 1.4.3, Part 7: a
    float mask is an additive bias; -inf is the forbidding value): same bits,
    including a row with every key forbidden (exactly zero)."""
    q, k, v, lens = _bias_case(2)
    B, H, Sq, Skv = q.shape[0], q.shape[1], q.shape[2], k.shape[2]
    m = _random_mask(310, (B, H, Sq, Skv))
    m[1, 2, 0, :] = False
    bias = np.where(m, 0.0, -np.inf)
    for causal in (0, 1):
        a, wa = attn(q, k, v, 0.6, causal, lens, mask=m, weights=True)
        b, wb = attn(q, k, v, 0.6, causal, lens, bias=bias, weights=True)
        assert np.array_equal(a, b) and np.array_equal(wa, wb), causal
        assert np.all(b[1, 2, 0] == 0.0)


def pin_row_constant_bias_changes_nothing(attn):
    """softmax is unchanged by one constant added to a whole row of logits:
    a bias that is constant along the keys (a different constant per row,
    head and batch item, up to +-50) leaves the output unchanged."""
    q, k, v, lens = _bias_case(3)
    B, H, Sq, Skv = q.shape[0], q.shape[1], q.shape[2], k.shape[2]
    c = 50.0 * (2.0 * np.random.default_rng(5).random((B, H, Sq, 1)) - 1.0)
    base = attn(q, k, v, 0.6, 1, lens)
    out = attn(q, k, v, 0.6, 1, lens, bias=np.broadcast_to(c, (B, H, Sq, Skv)))
    assert np.allclose(out, base, rtol=0, atol=1e-12)


def pin_bias_matches_torch_sdpa(attn):
    """Random finite biases in every broadcast shape, with the causal rule,
    valid lengths, grouped heads and a boolean mask, against torch's CPU
    scaled_dot_product_attention in float64 given the float attn_mask
    bias + (0 where allowed, -inf elsewhere) -- an independent routine that
    adds a float mask to the scaled logits."""
    import torch
    import torch.nn.functional as F
    for ci, shape in enumerate([(2, 4, 5, 7), (2, 1, 5, 7), (1, 4, 5, 7), (2, 4, 1, 7),
                                (1, 1, 5, 7)]):
        q, k, v, lens = _bias_case(10 + ci)
        B, H, Hkv, Sq, Skv = q.shape[0], q.shape[1], k.shape[1], q.shape[2], k.shape[2]
        bias = 3.0 * _rand(400 + ci, *shape)
        m = _random_mask(410 + ci, (B, 1, Sq, Skv), density=0.8) if ci % 2 else None
        causal = (ci // 2) % 2
        out, w = attn(q, k, v, 0.7, causal, lens, mask=m, bias=bias, weights=True)
        bb = np.broadcast_to(bias, (B, H, Sq, Skv))
        mm = np.ones((B, H, Sq, Skv), bool) if m is None else np.broadcast_to(m, (B, H, Sq, Skv))
        ke = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
        ve = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
        for b in range(B):
            rule, pad = _visible(Sq, Skv, causal, lens[b])
            for h in range(H):
                allowed = mm[b, h] & rule
                assert np.all(w[b, h][~allowed] == 0.0), (ci, b, h)
                rows = np.nonzero(allowed.any(axis=1))[0]
                assert np.all(out[b, h][~allowed.any(axis=1)] == 0.0), (ci, b, h)
                if len(rows) == 0:
                    continue
                fm = np.where(allowed, bb[b, h], -np.inf)[rows]
                ref = F.scaled_dot_product_attention(
                    torch.from_numpy(q[b, h, rows]), ke[b, h], ve[b, h],
                    attn_mask=torch.from_numpy(np.ascontiguousarray(fm)), scale=0.7).numpy()
                assert np.allclose(out[b, h, rows], ref, rtol=0, atol=1e-12), (ci, b, h)


def pin_low_precision_bias_widens_exactly(attn):
    """A bfloat16 or float32 bias is its exact float64 value: the same bits
    as the float64 call on the widened inputs."""
    q, k, v, lens = _bias_case(20)
    bias = 2.0 * _rand(420, 1, q.shape[1], q.shape[2], k.shape[2])
    ref = attn(*(bf16_to_f32(bf16_bits(x)).astype(np.float64) for x in (q, k, v)), 0.5, 1, lens,
               bias=bf16_to_f32(bf16_bits(bias)).astype(np.float64))
    got = attn(*(bf16_bits(x) for x in (q, k, v)), 0.5, 1, lens, bias=bf16_bits(bias))
    assert np.array_equal(got, ref)
    ref = attn(*(x.astype(np.float32).astype(np.float64) for x in (q, k, v)), 0.5, 1, lens,
               bias=bias.astype(np.float32).astype(np.float64))
    got = attn(*(x.astype(np.float32) for x in (q, k, v)), 0.5, 1, lens,
               bias=bias.astype(np.float32))
    assert np.array_equal(got, ref)


ALL_PINS = [
    pin_p2_causal_example,
    pin_p3_unmasked_example,
    pin_row_sums_and_forbidden_zero,
    pin_future_invariance,
    pin_zero_query_uniform,
    pin_convex_mixture,
    pin_shift_invariance_large_logits,
    pin_two_key_logistic,
    pin_matches_torch_sdpa,
    pin_decode_is_last_prefill_row,
    pin_key_permutation_equivariance,
    pin_low_precision_inputs_widen_exactly,
    pin_length_clamp,
    pin_grouped_heads_match_expansion,
    pin_mask_of_the_rules_equals_the_rules,
    pin_key_padding_mask_equals_lengths,
    pin_mask_single_allowed_key,
    pin_mask_matches_torch_sdpa,
    pin_zero_bias_is_no_bias,
    pin_neg_inf_bias_is_the_boolean_mask,
    pin_row_constant_bias_changes_nothing,
    pin_bias_matches_torch_sdpa,
    pin_low_precision_bias_widens_exactly,
]


def failing_pins(attn) -> list:
    """Names of the pins that fail (or raise) for ``attn``."""
    bad = []
    for pin in ALL_PINS:
        try:
            pin(attn)
        except Exception as exc:  # a crash counts as a failed pin
            bad.append((pin.__name__, f"{type(exc).__name__}: {str(exc)[:120]}"))
    return bad
