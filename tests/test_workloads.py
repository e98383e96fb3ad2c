"""The seeded input generator (CPU only)."""
import math

import numpy as np

import workloads as W


def test_bf16_rounding_is_nearest_even():
    # Compare against a direct search of the two neighbouring bf16 values,
    # over a sweep of float32 bit patterns that includes every tie.
    rng = np.random.default_rng(0)
    bits = np.concatenate([rng.integers(0, 2**31 - 2**23, 20000, dtype=np.uint32),
                           (np.arange(0, 2**16, dtype=np.uint32) << 8) | 0x3F800000,
                           np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32)])
    # finite, and below the top binade (where rounding up overflows to inf)
    bits = bits[(bits & 0x7FFFFFFF) < 0x7F000000]
    x = bits.view(np.float32)
    got = W.bf16_to_f32(W.bf16_bits(x)).astype(np.float64)
    lo = (bits & 0xFFFF0000).view(np.float32).astype(np.float64)
    hi = ((bits & 0xFFFF0000) + 0x10000).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dlo, dhi = np.abs(xd - lo), np.abs(hi - xd)
    lo_even = ((bits >> 16) & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    assert np.array_equal(got, want)


def test_slices_regenerate_identically():
    w = W.WORKLOADS["padded2048_bf16"]
    lens = W.kv_lens_for(w)
    small = W.Workload("t", 3, 4, 40, 40, 16, "bf16", True, 11, (5, 40))
    full = W.make_inputs(small)
    pairs = [(2, 1), (0, 3)]
    sub = W.make_inputs(small, pairs=pairs)
    for idx, (b, h) in enumerate(pairs):
        for t in ("q", "k", "v"):
            assert np.array_equal(sub[t][idx, 0], full[t][b, h])
    assert list(sub["kv_lens"]) == [full["kv_lens"][2], full["kv_lens"][0]]
    assert lens.min() >= 256 and lens.max() <= 2048
    # padded tails hold the fill value, valid rows are drawn
    L0 = int(full["kv_lens"][0])
    assert np.all(full["k"][0, :, L0:] == 0) and np.all(full["k"][0, :, :L0] != 0)


def test_lengths_are_seeded():
    w = W.WORKLOADS["decode8192_bf16"]
    a, b = W.kv_lens_for(w), W.kv_lens_for(w)
    assert np.array_equal(a, b) and a.min() >= 512 and a.max() <= 8192 and len(a) == 64


def test_dot_product_variance_and_scale():
    # KubeDojo "Attention from Scratch" (module 1.4.3), Part 2: with unit-variance entries the dot
    # product's variance is about d_k (64) and about 1 after the 1/sqrt(d_k)
    # scale; and "Scaled dot-product attention with masking" gives the scale
    # at d_k = 128 as about 0.088.
    w = W.Workload("var", 1, 1, 4096, 4096, 64, "f32", False, 0)
    q = W.make_tensor(w, "q")[0, 0].astype(np.float64)
    k = W.make_tensor(w, "k")[0, 0].astype(np.float64)
    dots = (q * k).sum(axis=1)
    assert abs(dots.var() / 64 - 1) < 0.06
    assert abs((dots * w.scale).var() - 1) < 0.06
    s128 = W.WORKLOADS["prefill4096_bf16"].scale
    assert round(s128, 3) == 0.088 and np.float32(s128) == np.float32(1 / math.sqrt(128))


def test_batch_item_inputs_match_whole_tensors():
    """The per-batch-item regeneration the full-size GPU checks use gives the
    same bits as drawing the whole tensors (grouped K/V heads, ragged lengths)."""
    from gpu_util import batch_item_inputs
    w = W.Workload("small_gqa", 3, 8, 20, 40, 16, "bf16", True, 5, (3, 40), Hkv=2)
    lens = W.kv_lens_for(w)
    full = {t: W.make_tensor(w, t, lens) for t in ("q", "k", "v")}
    for b in range(w.B):
        q, k, v = batch_item_inputs(w, b, lens)
        assert np.array_equal(q[0], full["q"][b])
        assert np.array_equal(k[0], full["k"][b])
        assert np.array_equal(v[0], full["v"][b])
