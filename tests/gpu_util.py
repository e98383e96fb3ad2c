"""Helpers for the GPU tests: run the library and the oracle on the same bits."""
from __future__ import annotations

import math

import numpy as np

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W

BF16_TOL = 2e-2   # max-abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs error, fp32 inputs


def key_groups(B, H, Sq, Skv, d, dv=None, dtype="bf16", masked=False, general=False):
    """Wave sets that split each prefill block's keys (1 or 2; 1 for every
    other kernel).  Two calls give the same bits only when they agree on it:
    two key groups sum each row's keys in another order."""
    if dtype != "bf16" or Sq == 1:
        return 1
    return attn.prefill_plan(B, H, Sq, Skv, d, dv, masked=masked, general=general)[2]


def gpu_run(q, k, v, scale, causal, kv_lens=None, device="cuda", **kw):
    """Upload numpy inputs (float32, or uint16 bf16 bits), run attn.fwd,
    return (out as float64 numpy, out tensor)."""
    import torch
    tq, tk, tv = (W.to_torch(x, device) for x in (q, k, v))
    tl = None if kv_lens is None else torch.as_tensor(np.asarray(kv_lens, dtype=np.int32)).to(device)
    out = attn.fwd(tq, tk, tv, causal=causal, kv_lens=tl, scale=scale, **kw)
    torch.cuda.synchronize()
    return W.from_torch(out), out


def pad_rows(B, Sq, Skv, kv_lens):
    """[B, Sq] bool: query rows that are padding under the length reading."""
    pad = np.zeros((B, Sq), dtype=bool)
    for b in range(B):
        L = Skv if kv_lens is None else min(max(int(kv_lens[b]), 0), Skv)
        pad[b, min(Sq, L):] = True
    return pad


def assert_matches(got, ref, tol, kv_lens=None, Skv=None, what=""):
    """Element-wise max-abs check, and exact zeros on padded query rows
    (rows i >= min(Sq, clamp(L_b, 0, Skv)))."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    worst = float(err.max()) if err.size else 0.0
    where = np.unravel_index(err.argmax(), err.shape) if err.size else None
    assert worst <= tol, f"{what}: max abs err {worst:.3g} > {tol} at {where}"
    if kv_lens is not None:
        pad = pad_rows(got.shape[0], got.shape[2], Skv, kv_lens)
        for b in range(got.shape[0]):
            assert np.all(got[b][:, pad[b]] == 0.0), f"{what}: padded rows of batch {b} not zero"
    return worst


def check_problem(prob, causal, tol, what=""):
    """Run one random_problem dict on GPU and oracle; compare element-wise."""
    q, k, v, lens, scale = prob["q"], prob["k"], prob["v"], prob["kv_lens"], prob["scale"]
    got, _ = gpu_run(q, k, v, scale, causal, lens)
    Skv = k.shape[2]
    clamped = None if lens is None else np.clip(lens, 0, Skv)
    ref = oracle.attention(q, k, v, scale, causal, clamped)
    return assert_matches(got, ref, tol, clamped, Skv, what)


_ITEM_CACHE = {}          # (workload, b) -> (q, k, v), oldest first
_ITEM_CACHE_BYTES = 24 << 30


def batch_item_inputs(w, b, lens):
    """Host bits of batch item b of workload w, regenerated from the seeds:
    q [1, H, Sq, d], and k, v [1, H_kv, Skv, d] (each K/V head drawn once).
    Items are kept (up to 24 GiB) for the other full-size checks of the same
    workload."""
    key = (w, b)
    if key in _ITEM_CACHE:
        return _ITEM_CACHE[key]
    item = _draw_batch_item(w, b, lens)
    _ITEM_CACHE[key] = item
    while sum(sum(x.nbytes for x in it) for it in _ITEM_CACHE.values()) > _ITEM_CACHE_BYTES:
        _ITEM_CACHE.pop(next(iter(_ITEM_CACHE)))
    return item


def _draw_batch_item(w, b, lens):
    g = w.H // w.kv_heads
    q = W.make_tensor(w, "q", lens, pairs=[(b, h) for h in range(w.H)])
    kv = [W.make_tensor(w, t, lens, pairs=[(b, j * g) for j in range(w.kv_heads)])
          for t in ("k", "v")]
    return (q.reshape(1, w.H, w.Sq, w.d),
            kv[0].reshape(1, w.kv_heads, w.Skv, w.d), kv[1].reshape(1, w.kv_heads, w.Skv, w.d))


def check_workload_full(w, mask_np=None, say=print, bias_np=None):
    """Run workload w whole on the GPU, in the benchmark's launch
    configuration (optionally with an allowed-mask), and compare every
    (b, h) slice of the output with the oracle, one batch item at a time; the
    oracle's inputs are regenerated from the seeds and checked to be the very
    bits the GPU consumed."""
    import torch
    say("workload", w.name, "full", "mask" if mask_np is not None else "", flush=True)
    x = W.device_inputs(w)
    out = attn.fwd(x["q"], x["k"], x["v"], causal=w.causal, kv_lens=x["kv_lens"],
                   scale=x["scale"], mask=None if mask_np is None else W.mask_to_torch(mask_np),
                   bias=None if bias_np is None else W.bias_to_torch(bias_np))
    torch.cuda.synchronize()
    lens = W.kv_lens_for(w)
    m_all = None if mask_np is None else np.broadcast_to(
        mask_np, (w.B, w.H, mask_np.shape[2], w.Skv))
    worst = 0.0
    for b in range(w.B):
        q, k, v = batch_item_inputs(w, b, lens)
        assert np.array_equal(W.bits_from_torch(x["q"][b]), q[0]), f"{w.name}: q bits of b={b}"
        assert np.array_equal(W.bits_from_torch(x["k"][b]), k[0]), f"{w.name}: k bits of b={b}"
        assert np.array_equal(W.bits_from_torch(x["v"][b]), v[0]), f"{w.name}: v bits of b={b}"
        lb = None if lens is None else np.asarray(lens[b:b + 1])
        bias_b = None
        if bias_np is not None:
            bias_b = bias_np[b:b + 1] if bias_np.shape[0] > 1 else bias_np
        ref = oracle.attention(q, k, v, x["scale"], int(w.causal), lb,
                               mask=None if m_all is None else m_all[b:b + 1], bias=bias_b)
        got = W.from_torch(out[b:b + 1])
        worst = max(worst, assert_matches(got, ref, BF16_TOL, lb, w.Skv, f"{w.name} b={b}"))
    say("workload", w.name, "max abs err over all slices", worst, flush=True)
    return worst
