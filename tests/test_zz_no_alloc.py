"""attn_fwd_noalloc against attn_fwd_ex on the GPU (MI355X).

attn_fwd_noalloc runs the kernels of attn_fwd_ex with its temporary memory
in the library's fixed per-device scratch array, so on the same inputs it
must give the same bits.  Each case makes two calls in a row, the second on
a smaller problem, since the array keeps the previous call's contents."""
import ctypes

import numpy as np
import pytest

import oracle
import transformer_scaled_dot_attn_amd as attn
import workloads as W
from gpu_util import BF16_TOL, assert_matches

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(fn_name, x, out, mask=None):
    """One call of attn_fwd_noalloc or attn_fwd_ex through the C ABI."""
    import torch
    lib = attn.library()
    q, k, v = x["q"], x["k"], x["v"]
    B, H, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    mp, sb, sh, si = (None, 0, 0, 0) if mask is None else attn._mask(mask, B, H, Sq, Skv, q.device)
    stream = torch.cuda.current_stream().cuda_stream
    common = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Hkv, Sq, Skv, d, d,
              ctypes.c_float(x["scale"]), int(x["causal"]), _ptr(x["lens"]), mp, sb, sh, si,
              attn.BF16, stream]
    if fn_name == "noalloc":
        return lib.attn_fwd_noalloc(*common)
    return lib.attn_fwd_ex(*common, None, 0)


def _problem(seed, B, H, Hkv, Sq, Skv, d, causal, lens):
    import torch
    w = W.Workload("noalloc", B, H, Sq, Skv, d, "bf16", causal, seed, Hkv=Hkv)
    lt = None if lens is None else np.asarray(lens, np.int32)
    host = {t: W.make_tensor(w, t, lt) for t in ("q", "k", "v")}
    x = {t: W.to_torch(host[t], "cuda") for t in host}
    x["lens"] = None if lt is None else torch.as_tensor(lt).to("cuda")
    x["scale"], x["causal"], x["host"], x["lens_host"] = w.scale, causal, host, lt
    return x


# (label, first problem, second smaller problem); each problem is
# (seed, B, H, H_kv, Sq, Skv, d, causal, lengths, mask kind)
CASES = [
    ("decode", (1, 4, 8, 2, 1, 3000, 128, False, [3000, 17, 2100, 0], None),
     (2, 2, 4, 4, 1, 500, 128, False, [500, 33], None)),
    ("decode d64 MQA", (3, 3, 32, 1, 1, 4100, 64, False, [4100, 1, 2000], None),
     (4, 1, 8, 1, 1, 700, 64, False, [650], None)),
    ("split prefill", (5, 1, 8, 8, 300, 6000, 128, True, None, None),
     (6, 1, 4, 2, 100, 3000, 128, True, None, None)),
    ("masked decode", (7, 3, 8, 4, 1, 2000, 128, False, [2000, 900, 31], "random"),
     (8, 2, 4, 4, 1, 300, 128, False, [300, 120], "random")),
    ("masked prefill", (9, 2, 4, 4, 512, 512, 128, True, [512, 300], "padding"),
     (10, 1, 2, 2, 200, 260, 64, True, None, "padding")),
    ("prefill without temporary memory", (11, 2, 4, 4, 300, 300, 128, True, [300, 111], None),
     (12, 1, 2, 1, 70, 70, 64, True, None, None)),
]


def _mask_for(kind, B, H, Sq, Skv, seed):
    if kind is None:
        return None, None
    if kind == "random":
        m = W.random_mask(seed, (B, H, 1, Skv), 0.6)
    else:
        m = W.key_padding_mask([min(7, Skv - 1)] * B, [Skv] * B, Skv)
    return m, W.mask_to_torch(m)


@pytest.mark.parametrize("label,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_attn_fwd_ex(label, first, second):
    import torch
    for n, (seed, B, H, Hkv, Sq, Skv, d, causal, lens, mk) in enumerate((first, second)):
        _say(f"noalloc {label} call {n + 1}: B={B} H={H} H_kv={Hkv} Sq={Sq} Skv={Skv} d={d} "
             f"mask={mk}")
        x = _problem(seed, B, H, Hkv, Sq, Skv, d, causal, lens)
        mhost, mask = _mask_for(mk, B, H, Sq, Skv, seed)
        need = attn.workspace_bytes(B, H, Sq, Skv, d, attn.BF16, kv_heads=Hkv,
                                    masked=mask is not None)
        assert need <= attn.noalloc_scratch_bytes()
        out_a = torch.full((B, H, Sq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        out_b = torch.full_like(out_a, float("nan"))
        assert _call("noalloc", x, out_a, mask) == attn.OK
        assert _call("ex", x, out_b, mask) == attn.OK
        torch.cuda.synchronize()
        a, b = W.bits_from_torch(out_a), W.bits_from_torch(out_b)
        assert np.array_equal(a, b), f"{label} call {n + 1}: attn_fwd_noalloc bits differ"
        if n == 1:
            # the second call also against the oracle, to the bf16 tolerance
            ref = oracle.attention(x["host"]["q"], x["host"]["k"], x["host"]["v"], x["scale"],
                                   int(causal), x["lens_host"], mask=mhost)
            got = W.from_torch(out_a)
            clamped = None if lens is None else np.clip(lens, 0, Skv)
            assert_matches(got, ref, BF16_TOL, clamped, Skv, f"{label} vs oracle")
