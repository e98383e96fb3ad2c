"""Structural properties of the GPU kernels that hold at any size (MI355X).

These need no oracle: each compares the library with itself under a change
the method says must (or must not) matter."""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, gpu_run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bits(t):
    return W.bits_from_torch(t)


@pytest.mark.parametrize("Sq,Skv,d,causal,lens", [
    (300, 300, 128, 1, [300, 137, 1]),   # prefill, padded
    (90, 400, 64, 1, [350, 200, 91]),    # fewer queries than keys
    (1, 3000, 128, 0, [3000, 1000, 1]),  # decode
])
def test_padding_is_never_read(Sq, Skv, d, causal, lens):
    """NaN in padded key/value rows and padded query rows changes nothing:
    the output is bitwise identical to the zero-filled run."""
    import torch
    _say("poison", Sq, Skv, d, causal, lens)
    B, H = len(lens), 2
    w = W.Workload("poison", B, H, Sq, Skv, d, "bf16", bool(causal), 77)
    outs = []
    for fill in (0.0, float("nan")):
        lt = np.array(lens, np.int32)
        q = W.make_tensor(w, "q", lt, pad_fill=fill)
        k = W.make_tensor(w, "k", lt, pad_fill=fill)
        v = W.make_tensor(w, "v", lt, pad_fill=fill)
        _, out = gpu_run(q, k, v, w.scale, causal, lt)
        outs.append(_bits(out))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("d", [64, 128])
def test_future_keys_do_not_leak(d):
    """Changing keys/values at positions >= t leaves query rows < t bitwise
    unchanged under the causal mask."""
    S = 333
    prob = W.random_problem(5, 1, 2, S, S, d, "bf16")
    _, base = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    base = _bits(base)
    rng = np.random.default_rng(1)
    for t in (1, 63, 64, 65, 128, 200, 332):
        k, v = prob["k"].copy(), prob["v"].copy()
        k[:, :, t:] = W.bf16_bits(rng.standard_normal(k[:, :, t:].shape, dtype=np.float32) * 4)
        v[:, :, t:] = W.bf16_bits(rng.standard_normal(v[:, :, t:].shape, dtype=np.float32) * 4)
        _, out = gpu_run(prob["q"], k, v, prob["scale"], 1)
        out = _bits(out)
        assert np.array_equal(out[:, :, :t], base[:, :, :t]), f"rows < {t} changed"


def test_first_causal_row_is_first_value_row():
    """Row 0 sees only key 0, so its output is V[0] exactly."""
    prob = W.random_problem(6, 2, 3, 150, 150, 128, "bf16")
    _, out = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    assert np.array_equal(_bits(out)[:, :, 0], prob["v"][:, :, 0])
    prob = W.random_problem(6, 1, 1, 16, 16, 16, "f32")
    _, out = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    assert np.array_equal(_bits(out)[:, :, 0], prob["v"][:, :, 0].view(np.uint32))


def test_zero_queries_give_prefix_means():
    """Q = 0 gives uniform weights: row i is the mean of V[0..i]."""
    B, H, S, d = 1, 2, 200, 128
    prob = W.random_problem(7, B, H, S, S, d, "bf16")
    q = np.zeros_like(prob["q"])
    got, _ = gpu_run(q, prob["k"], prob["v"], prob["scale"], 1)
    vv = W.bf16_to_f32(prob["v"]).astype(np.float64)
    ref = np.cumsum(vv, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.abs(got - ref).max() <= BF16_TOL


def test_decode_matches_last_prefill_row():
    """One decode query against the cache equals the last row of causal
    prefill over the same keys (cached and uncached generation agree)."""
    B, H, S, d = 2, 4, 777, 128
    prob = W.random_problem(8, B, H, S, S, d, "bf16")
    lens = [777, 500]
    full, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1, lens)
    for b, L in enumerate(lens):
        qd = np.ascontiguousarray(prob["q"][b:b + 1, :, L - 1:L])
        dec, _ = gpu_run(qd, prob["k"][b:b + 1], prob["v"][b:b + 1], prob["scale"], 0, [L])
        assert np.abs(dec[0, :, 0] - full[b, :, L - 1]).max() <= BF16_TOL
        dec1, _ = gpu_run(qd, prob["k"][b:b + 1], prob["v"][b:b + 1], prob["scale"], 1, [L])
        assert np.array_equal(dec1, dec), "the causal flag must not matter for one query"


def test_heads_and_batches_are_independent():
    """Permuting heads (and batch items) permutes the outputs bitwise."""
    prob = W.random_problem(9, 2, 4, 130, 130, 64, "bf16", [130, 77])
    _, out = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1, [130, 77])
    hp, bp = [3, 1, 0, 2], [1, 0]
    q = np.ascontiguousarray(prob["q"][bp][:, hp])
    k = np.ascontiguousarray(prob["k"][bp][:, hp])
    v = np.ascontiguousarray(prob["v"][bp][:, hp])
    _, out2 = gpu_run(q, k, v, prob["scale"], 1, [77, 130])
    assert np.array_equal(_bits(out2), _bits(out)[bp][:, hp])


def test_caller_workspace_and_streams():
    """attn_fwd_ws with a caller buffer, and a call on a side stream, give
    the bits of attn_fwd; a short buffer is refused."""
    import torch
    prob = W.random_problem(10, 3, 4, 1, 2500, 128, "bf16", [2500, 10, 1900])
    q, k, v = (W.to_torch(prob[x]) for x in ("q", "k", "v"))
    lens = torch.tensor([2500, 10, 1900], dtype=torch.int32, device="cuda")
    ref = attn.fwd(q, k, v, kv_lens=lens, causal=False)
    nbytes = attn.workspace_bytes(3, 4, 1, 2500, 128, attn.BF16)
    # a caller's workspace needs no initialisation: fill it with garbage
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    out = attn.fwd(q, k, v, kv_lens=lens, causal=False, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out2 = attn.fwd(q, k, v, kv_lens=lens, causal=False, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))
    with pytest.raises(attn.AttnError) as e:
        attn.fwd(q, k, v, kv_lens=lens, causal=False, workspace=ws[: nbytes - 256])
    assert e.value.status == attn.E_WORKSPACE


def test_all_lengths_zero():
    prob = W.random_problem(11, 2, 2, 64, 64, 128, "bf16", [0, 0])
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1, [0, 0])
    assert np.all(got == 0.0)
    prob = W.random_problem(11, 2, 2, 1, 64, 128, "bf16", [0, 0])
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, [0, 0])
    assert np.all(got == 0.0)


def test_repeat_runs_are_bitwise_stable():
    prob = W.random_problem(12, 1, 32, 1024, 1024, 128, "bf16")
    _, a = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    _, b = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 1)
    assert np.array_equal(_bits(a), _bits(b))


def test_library_workspace_per_stream():
    """Two decodes enqueued on two streams with the library-owned workspace
    (attn_fwd with no workspace argument) run concurrently without sharing
    temporary memory: each gives the bits of the same call run alone."""
    import torch
    probs = [W.random_problem(13 + i, 4, 8, 1, 3000, 128, "bf16", [3000, 1500, 2999, 700])
             for i in range(2)]
    lens = torch.tensor([3000, 1500, 2999, 700], dtype=torch.int32, device="cuda")
    xs = [[W.to_torch(p[x]) for x in ("q", "k", "v")] for p in probs]
    alone = []
    for q, k, v in xs:
        alone.append(attn.fwd(q, k, v, kv_lens=lens, causal=False))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(a) for a in alone]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(20):
        for (q, k, v), s, o in zip(xs, streams, outs):
            with torch.cuda.stream(s):
                attn.fwd(q, k, v, o, kv_lens=lens, causal=False)
    torch.cuda.synchronize()
    for o, a in zip(outs, alone):
        assert torch.equal(o.view(torch.int16), a.view(torch.int16))


def test_decode_repeats_with_split_prefills_between():
    """Repeated decodes on the library workspace give identical bits, also
    with split prefills (whose partials share that workspace) between them."""
    import torch
    dec = W.random_problem(60, 6, 8, 1, 5000, 128, "bf16", [5000, 4000, 33, 0, 4999, 1200],
                           Hkv=2)
    pre = W.random_problem(61, 1, 8, 300, 6000, 128, "bf16")
    dq, dk, dv = (W.to_torch(dec[x]) for x in ("q", "k", "v"))
    pq, pk, pv = (W.to_torch(pre[x]) for x in ("q", "k", "v"))
    lens = torch.as_tensor(np.asarray(dec["kv_lens"], np.int32)).to("cuda")
    assert attn.workspace_bytes(1, 8, 300, 6000, 128, attn.BF16) > 0   # key-range splits
    first = attn.fwd(dq, dk, dv, kv_lens=lens, causal=False)
    base = _bits(first)
    ref = oracle.attention(dec["q"], dec["k"], dec["v"], dec["scale"], 0, dec["kv_lens"])
    assert np.abs(W.from_torch(first) - ref).max() <= BF16_TOL
    for rep in range(6):
        if rep % 2:
            attn.fwd(pq, pk, pv, causal=True)
        out = attn.fwd(dq, dk, dv, kv_lens=lens, causal=False)
        assert np.array_equal(_bits(out), base), f"repeat {rep}"


def test_decode_many_caches():
    """A decode over 66560 (b, K/V head) caches of up to 33 keys, some empty."""
    B, H, Skv, d = 1040, 64, 33, 64
    rng = np.random.default_rng(62)
    lens = rng.integers(0, Skv + 1, size=B).astype(np.int32)
    prob = W.random_problem(62, B, H, 1, Skv, d, "bf16", lens)
    got, _ = gpu_run(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    ref = oracle.attention(prob["q"], prob["k"], prob["v"], prob["scale"], 0, lens)
    from gpu_util import assert_matches
    assert_matches(got, ref, BF16_TOL, lens, Skv, "66560 caches")
