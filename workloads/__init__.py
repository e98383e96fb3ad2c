"""Seeded synthetic inputs shaped like the pages' attention workloads.

This module holds no attention arithmetic.  It draws Q, K, V and per-sequence
valid lengths from fixed seeds and stores them as float32 or as bfloat16 bit
patterns (uint16, round-to-nearest-even from the float32 draw).  Both the GPU
tests and the CPU oracle consume exactly these bits.

Recipe (every draw uses numpy's PCG64 through ``default_rng``):
  * valid lengths: ``default_rng(SeedSequence([seed, 0]))``, then
    ``integers(lo, hi + 1, size=B)``, i.e. uniform on [lo, hi] inclusive;
  * each (tensor t, batch b, head h) slice has its own stream
    ``default_rng(SeedSequence([seed, t, b, h]))`` with t = 1, 2, 3 for
    q, k, v; it draws ``standard_normal((rows, d), float32)`` for the slice's
    valid rows only -- the first n_b query rows and the first L_b key/value
    rows, where n_b = min(Sq, L_b) -- so any slice can be regenerated on its
    own and the padded tail is never drawn;
  * padded rows hold ``pad_fill`` (0.0 by default; NaN for poison tests).
Values are i.i.d. N(0, 1), as the pages' torch.randn examples are.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Sequence

import numpy as np

TENSOR_IDS = {"q": 1, "k": 2, "v": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem.  Sizes follow [B, H, S, d] layout."""
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    d: int
    dtype: str              # "f32" or "bf16"
    causal: bool
    seed: int
    kv_len_range: Optional[tuple] = None   # (lo, hi) inclusive, or None
    description: str = ""
    Hkv: Optional[int] = None              # key/value heads (None: H, multi-head)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32, returned as that float32's value."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The pages' shapes: d_model 4096 = 32 heads of 128 ("Attention from First
# Principles", section 5; "Scaled dot-product attention with masking",
# "Multi-head attention"), d_k = 64 ("Attention from Scratch", KubeDojo module 1.4.3, the scale-factor
# discussion), prefill S = 2048 against decode over a KV cache ("Attention from
# First Principles", section 6), and small seeded randn fixtures.
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 1, 1, 64, 64, 16, "f32", True, 1,
                 description="causal single head, S=64, d=16, fp32"),
        Workload("mha768_bf16", 4, 12, 512, 512, 64, "bf16", True, 2,
                 description="causal MHA, d_model=768 (12x64), S=512"),
        Workload("prefill4096_bf16", 1, 32, 4096, 4096, 128, "bf16", True, 3,
                 description="causal MHA prefill, d_model=4096 (32x128), S=4096"),
        Workload("padded2048_bf16", 8, 32, 2048, 2048, 128, "bf16", True, 4, (256, 2048),
                 description="causal + right padding, S=2048, lengths U[256,2048]"),
        Workload("decode8192_bf16", 64, 32, 1, 8192, 128, "bf16", False, 5, (512, 8192),
                 description="decode, one query against a KV cache of capacity 8192, "
                             "lengths U[512,8192]"),
        # Grouped K/V heads at the GQA(8) shape of the Llama-3-8B example, 32
        # query heads and 8 K/V heads ("Attention from First Principles",
        # section 7), and MQA (one K/V head): the h_kv in {1, 8, 32} sweep of
        # that page's section 10, exercise F.
        Workload("gqa_prefill2048_bf16", 2, 32, 2048, 2048, 128, "bf16", True, 6, Hkv=8,
                 description="causal GQA prefill, 32 query heads over 8 K/V heads, S=2048"),
        Workload("gqa_decode8192_bf16", 64, 32, 1, 8192, 128, "bf16", False, 7, (512, 8192),
                 Hkv=8, description="GQA decode, 32 query heads over 8 K/V heads, capacity "
                                    "8192, lengths U[512,8192]"),
        Workload("mqa_decode8192_bf16", 64, 32, 1, 8192, 128, "bf16", False, 8, (512, 8192),
                 Hkv=1, description="MQA decode, 32 query heads over one K/V head, capacity "
                                    "8192, lengths U[512,8192]"),
    ]
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def kv_lens_for(w: Workload) -> Optional[np.ndarray]:
    if w.kv_len_range is None:
        return None
    lo, hi = w.kv_len_range
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0]))
    return rng.integers(lo, hi + 1, size=w.B).astype(np.int32)


def _slice(seed: int, tensor: str, b: int, h: int, rows: int, d: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, TENSOR_IDS[tensor], b, h]))
    return rng.standard_normal((rows, d), dtype=np.float32)


def _valid_rows(w: Workload, lens: Optional[np.ndarray], b: int, tensor: str) -> int:
    L = w.Skv if lens is None else int(min(max(int(lens[b]), 0), w.Skv))
    if tensor == "q":
        return min(w.Sq, L)
    return L


def make_tensor(w: Workload, tensor: str, lens: Optional[np.ndarray] = None,
                pairs: Optional[Iterable[tuple]] = None, pad_fill: float = 0.0) -> np.ndarray:
    """Draw one of q/k/v.  Returns float32 [B,H,S,d] for "f32" workloads and
    uint16 bf16 bits for "bf16" (k and v have the workload's K/V head count).
    With ``pairs`` (an iterable of (b, h) query heads), only those slices are
    drawn -- for k and v, the slice of each pair's K/V head h // (H // H_kv)
    -- and the result is [len(pairs), 1, S, d]."""
    S = w.Sq if tensor == "q" else w.Skv
    heads = w.H if tensor == "q" else w.kv_heads
    group = w.H // w.kv_heads
    out_dtype = np.float32 if w.dtype == "f32" else np.uint16
    if pairs is None:
        sel = [(b, h) for b in range(w.B) for h in range(heads)]
        shape = (w.B, heads, S, w.d)
    else:
        # pairs name query heads; key/value slices are those of their K/V head
        sel = [(b, h if tensor == "q" else h // group) for b, h in pairs]
        shape = (len(sel), 1, S, w.d)
    if w.dtype == "f32":
        fill = np.float32(pad_fill)
    else:
        fill = bf16_bits(np.array([pad_fill], dtype=np.float32))[0]
    out = np.empty(shape, dtype=out_dtype)
    flat = out.reshape(-1, S, w.d)
    for idx, (b, h) in enumerate(sel):
        rows = _valid_rows(w, lens, b, tensor)
        x = _slice(w.seed, tensor, b, h, rows, w.d)
        flat[idx, :rows] = x if w.dtype == "f32" else bf16_bits(x)
        flat[idx, rows:] = fill
    return out


def make_inputs(w: Workload, pairs: Optional[Sequence[tuple]] = None,
                pad_fill: float = 0.0) -> dict:
    """All inputs of a workload: q, k, v (see ``make_tensor``), kv_lens (int32
    [B] or None; restricted to the chosen pairs' batch items when ``pairs`` is
    given) and scale."""
    lens = kv_lens_for(w)
    q = make_tensor(w, "q", lens, pairs, pad_fill)
    k = make_tensor(w, "k", lens, pairs, pad_fill)
    v = make_tensor(w, "v", lens, pairs, pad_fill)
    sub_lens = lens
    if pairs is not None and lens is not None:
        sub_lens = np.array([lens[b] for b, _ in pairs], dtype=np.int32)
    return {"q": q, "k": k, "v": v, "kv_lens": sub_lens, "scale": w.scale, "workload": w}


def random_problem(seed: int, B: int, H: int, Sq: int, Skv: int, d: int, dtype: str = "f32",
                   kv_lens: Optional[Sequence[int]] = None, dv: Optional[int] = None,
                   Hkv: Optional[int] = None) -> dict:
    """A small ad-hoc problem with every row drawn (pad rows included): used by
    tests that sweep many shapes.  dtype "f64", "f32" or "bf16" (uint16 bits);
    k and v have Hkv heads (default H)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 99]))
    dv = d if dv is None else dv
    Hkv = H if Hkv is None else Hkv
    q = rng.standard_normal((B, H, Sq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Skv, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Skv, dv), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    elif dtype == "f64":
        q, k, v = (x.astype(np.float64) for x in (q, k, v))
    lens = None if kv_lens is None else np.asarray(kv_lens, dtype=np.int32)
    return {"q": q, "k": k, "v": v, "kv_lens": lens,
            "scale": float(np.float32(1.0 / math.sqrt(d)))}


# ---- allowed-masks (inputs: True = may attend) ----------------------------
def random_mask(seed: int, shape: Sequence[int], density: float = 0.5) -> np.ndarray:
    """Bernoulli(density) bool mask of `shape` (last axis the keys), drawn as
    ``default_rng(SeedSequence([seed, 4])).random(shape) < density``."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4]))
    return rng.random(tuple(shape)) < density


def key_padding_mask(starts: Sequence[int], ends: Sequence[int], Skv: int) -> np.ndarray:
    """[B, 1, 1, Skv] key-padding mask: key j of sequence b is allowed iff
    starts[b] <= j < ends[b] (left padding before starts[b], right padding
    from ends[b]), the padding masks of a batch of unequal sources."""
    j = np.arange(Skv)[None, :]
    m = (j >= np.asarray(starts)[:, None]) & (j < np.asarray(ends)[:, None])
    return m[:, None, None, :]


def document_mask(doc_lens: Sequence[int]) -> np.ndarray:
    """[1, 1, S, S] mask of packed documents: row i may see key j iff both lie
    in the same document (consecutive runs of the given lengths, S their sum)."""
    doc = np.repeat(np.arange(len(doc_lens)), doc_lens)
    return (doc[:, None] == doc[None, :])[None, None]


def window_mask(S: int, width: int) -> np.ndarray:
    """[1, 1, S, S] sliding-window mask: row i may see keys i - width < j <= i + width
    (the causal flag then keeps the keys up to i)."""
    i = np.arange(S)
    return (np.abs(i[:, None] - i[None, :]) < width)[None, None]


def mask_to_torch(m: np.ndarray, device="cuda"):
    """bool mask -> a torch.bool view on `device` whose rows are stored in
    round_up(Skv, 4) bytes (the word-readable layout the library needs)."""
    import torch
    Skv = m.shape[-1]
    pad = (Skv + 3) // 4 * 4
    full = np.zeros(m.shape[:-1] + (pad,), dtype=bool)
    full[..., :Skv] = m
    return torch.from_numpy(full).to(device)[..., :Skv]


def random_bias(seed: int, shape: Sequence[int], dtype: str = "bf16", spread: float = 2.0,
                hide: float = 0.0) -> np.ndarray:
    """Additive bias of `shape` (last axis the keys): spread * N(0, 1) drawn
    as ``default_rng(SeedSequence([seed, 5])).standard_normal(shape,
    float32)``, with a fraction `hide` of the entries (drawn from the same
    stream) set to -inf; float32, or bf16 bits (RNE)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5]))
    x = spread * rng.standard_normal(tuple(shape), dtype=np.float32)
    if hide > 0.0:
        x[rng.random(tuple(shape)) < hide] = -np.inf
    return x if dtype == "f32" else bf16_bits(x)


def bias_to_torch(b: np.ndarray, device="cuda"):
    """float32 or bf16-bit bias -> a tensor view on `device` whose rows are
    stored in round_up(Skv, 4) elements (the 4-element groups the library
    reads)."""
    import torch
    Skv = b.shape[-1]
    pad = (Skv + 3) // 4 * 4
    full = np.zeros(b.shape[:-1] + (pad,), dtype=b.dtype)
    full[..., :Skv] = b
    return to_torch(full, device)[..., :Skv]


# ---- moving inputs to and from a GPU (torch only moves the bits) ----------
def to_torch(x: np.ndarray, device="cuda"):
    """float32 array -> float32 tensor; uint16 bf16 bits -> bfloat16 tensor."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    if x.dtype == np.float32:
        return torch.from_numpy(x).to(device)
    raise ValueError(f"cannot upload dtype {x.dtype}")


def from_torch(t) -> np.ndarray:
    """bfloat16 or float32 tensor -> the same values as a float64 array."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_to_f32(bits).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def bits_from_torch(t) -> np.ndarray:
    """Raw stored bits of a bfloat16 (uint16) or float32 (uint32) tensor."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def device_inputs(w: Workload, device="cuda", pad_fill: float = 0.0, digest: bool = False) -> dict:
    """The workload's q, k, v as device tensors, drawn and uploaded one batch
    item at a time (bounded host memory), plus kv_lens (device int32 or None),
    the host copy of the lengths, and scale.  With ``digest``, also "sha256":
    the SHA-256 of the q, k and v bytes as uploaded (row-major [B,H,S,d], one
    tensor after the other) followed by the int32 lengths, if any."""
    import hashlib
    import torch
    h = hashlib.sha256() if digest else None
    lens = kv_lens_for(w)
    tdtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    res = {}
    group = w.H // w.kv_heads
    for name, S in (("q", w.Sq), ("k", w.Skv), ("v", w.Skv)):
        heads = w.H if name == "q" else w.kv_heads
        t = torch.empty((w.B, heads, S, w.d), dtype=tdtype, device=device)
        for b in range(w.B):
            # one query head per K/V head selects that K/V head's slice
            pairs = [(b, h * (1 if name == "q" else group)) for h in range(heads)]
            part = make_tensor(w, name, lens, pairs=pairs, pad_fill=pad_fill)
            if h is not None:
                h.update(memoryview(np.ascontiguousarray(part)).cast("B"))
            t[b].copy_(to_torch(part.reshape(heads, S, w.d), device))
        res[name] = t
    if h is not None:
        if lens is not None:
            h.update(np.ascontiguousarray(lens, dtype=np.int32).tobytes())
        res["sha256"] = h.hexdigest()
    res["kv_lens"] = None if lens is None else torch.from_numpy(lens).to(device)
    res["kv_lens_host"] = lens
    res["scale"] = w.scale
    return res
