"""Helpers for the GPU tests: run the library and the oracle on the same bits."""
from __future__ import annotations

import math

import numpy as np

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W

BF16_TOL = 2e-2   # max-abs error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs error, fp32 inputs


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
