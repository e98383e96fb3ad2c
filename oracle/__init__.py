"""Float64 CPU oracle for scaled dot-product attention -- test infrastructure.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  It never imports the GPU library and the GPU library never
imports it; the two share no code.  The arithmetic lives in ``attn_oracle.c``
(plain C, float64, one thread per (batch, head) pair), which this module
compiles with gcc and calls through ctypes.

``attention`` follows the plain definition softmax(scale*QK^T + M) V with the
mask added before the softmax ("Self-Attention" notes, sections "Scaled
Dot-Product Attention" and "Causal Masking"; "Attention from First
Principles", section 4).  See the header of ``attn_oracle.c`` for the readings
taken where the pages leave a step open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_CODES = {np.dtype(np.float64): 0, np.dtype(np.float32): 1, np.dtype(np.uint16): 2}
ERRORS = {1: "null pointer", 2: "bad shape", 4: "bad dtype", 7: "non-finite scale",
          9: "out of memory"}


def compile_oracle(src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``src`` into the shared object ``out`` (no -ffast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def compile_oracle_sanitized(out: str, src: str = _SRC) -> str:
    """Compile the oracle with clang under AddressSanitizer and
    UndefinedBehaviorSanitizer (same language and floating-point flags), for
    the sanitizer job of the CPU tests; it needs the clang ASan runtime
    preloaded."""
    cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> str:
    """(Re)compile the oracle library in place."""
    return compile_oracle()


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    p, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.oracle_attn_fwd.argtypes = [p, p, p, i, p, i, i, i, i, i, i, d, i, p, i]
    lib.oracle_attn_fwd.restype = i
    lib.oracle_attn_fwd_weights.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, d, i, p, i]
    lib.oracle_attn_fwd_weights.restype = i
    lib.oracle_attn_fwd_gqa.argtypes = [p, p, p, i, p, i, i, i, i, i, i, i, d, i, p, i]
    lib.oracle_attn_fwd_gqa.restype = i
    lib.oracle_attn_fwd_weights_gqa.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, d, i, p,
                                                i]
    lib.oracle_attn_fwd_weights_gqa.restype = i
    ll = ctypes.c_longlong
    lib.oracle_attn_fwd_mask.argtypes = [p, p, p, i, p, i, i, i, i, i, i, i, d, i, p, p, ll, ll, i]
    lib.oracle_attn_fwd_mask.restype = i
    lib.oracle_attn_fwd_weights_mask.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, d, i, p, p,
                                                 ll, ll, i]
    lib.oracle_attn_fwd_weights_mask.restype = i
    lib.oracle_attn_fwd_ex.argtypes = [p, p, p, i, p, p, i, i, i, i, i, i, i, d, i, p, p, ll, ll,
                                       p, ll, ll, i]
    lib.oracle_attn_fwd_ex.restype = i
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = i
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library; builds it first when it is missing or stale.

    With ``path`` given, loads that file instead (used to load planted-mistake
    builds in the oracle's own tests)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB)
                    or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                compile_oracle()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def default_threads() -> int:
    return load().oracle_default_threads()


def attention(q, k, v, scale, causal, kv_lens=None, *, mask=None, bias=None, weights=False,
              nthreads=0, lib=None):
    """Reference attention forward.

    q: [B,H,Sq,d], k: [B,Hkv,Skv,d], v: [B,Hkv,Skv,dv] numpy arrays of one
    dtype: float64, float32, or uint16 holding bfloat16 bit patterns (widened
    exactly).  Hkv = H is multi-head attention; a divisor Hkv of H groups the
    query heads (query head h reads key/value head h // (H // Hkv)).
    scale: the multiplier of QK^T (a float; pass float32 values widened).
    kv_lens: None or int array [B] of valid lengths (clamped to [0, Skv]).
    mask: None or an array broadcastable to [B,H,Sq,Skv]; nonzero where query
    row i of (b, h) may see key j (combined with the causal and length rules
    by logical AND).  It is expanded to the full [B,H,Sq,Skv] bytes here.
    bias: None or an array of q's dtype broadcastable to [B,H,Sq,Skv], added
    to the scaled logits before the softmax; -inf forbids the key.
    Returns out [B,H,Sq,dv] float64, and with weights=True also the weight
    tensor [B,H,Sq,Skv].
    """
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODES:
        raise ValueError(f"q, k, v must share one of {list(DTYPE_CODES)}; got "
                         f"{q.dtype}, {k.dtype}, {v.dtype}")
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,S,d]")
    B, H, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    dv = v.shape[3]
    if k.shape != (B, Hkv, Skv, d) or v.shape[:3] != (B, Hkv, Skv):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"query heads {H} are not a multiple of key/value heads {Hkv}")
    lens_arr = None
    lens_ptr = None
    if kv_lens is not None:
        lens_arr = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int64).clip(-2**31, 2**31 - 1)
                                        .astype(np.int32))
        if lens_arr.shape != (B,):
            raise ValueError("kv_lens must have shape [B]")
        lens_ptr = lens_arr.ctypes.data
    out = np.empty((B, H, Sq, dv), dtype=np.float64)
    code = DTYPE_CODES[q.dtype]
    if bias is not None:
        bias = np.asarray(bias)
        if bias.dtype != q.dtype:
            raise ValueError(f"bias must have q's dtype {q.dtype}, got {bias.dtype}")
        if bias.ndim != 4 or bias.shape[3] != Skv:
            raise ValueError(f"bias must be 4-D [B|1, H|1, Sq|1, {Skv}]")
        # batch and head axes of size 1 stay broadcast (stride 0); rows are expanded
        Bb, Hb = bias.shape[0], bias.shape[1]
        bfull = np.ascontiguousarray(np.broadcast_to(bias, (Bb, Hb, Sq, Skv)))
        m = None if mask is None else np.ascontiguousarray(
            np.broadcast_to(np.asarray(mask) != 0, (B, H, Sq, Skv)), dtype=np.uint8)
        w = np.empty((B, H, Sq, Skv), dtype=np.float64) if weights else None
        rc = lib.oracle_attn_fwd_ex(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, code, out.ctypes.data,
            None if w is None else w.ctypes.data, B, H, Hkv, Sq, Skv, d, dv, float(scale),
            int(bool(causal)), lens_ptr, None if m is None else m.ctypes.data, H * Sq * Skv,
            Sq * Skv, bfull.ctypes.data, 0 if Bb == 1 else Hb * Sq * Skv, 0 if Hb == 1 else Sq * Skv,
            int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle error {rc}: {ERRORS.get(rc, 'unknown')}")
        return (out, w) if weights else out
    if mask is not None:
        m = np.ascontiguousarray(np.broadcast_to(np.asarray(mask) != 0, (B, H, Sq, Skv)),
                                 dtype=np.uint8)
        sb, sh = H * Sq * Skv, Sq * Skv
        if weights:
            w = np.empty((B, H, Sq, Skv), dtype=np.float64)
            rc = lib.oracle_attn_fwd_weights_mask(
                q.ctypes.data, k.ctypes.data, v.ctypes.data, code, out.ctypes.data, w.ctypes.data,
                B, H, Hkv, Sq, Skv, d, dv, float(scale), int(bool(causal)), lens_ptr,
                m.ctypes.data, sb, sh, int(nthreads))
        else:
            rc = lib.oracle_attn_fwd_mask(
                q.ctypes.data, k.ctypes.data, v.ctypes.data, code, out.ctypes.data, B, H, Hkv, Sq,
                Skv, d, dv, float(scale), int(bool(causal)), lens_ptr, m.ctypes.data, sb, sh,
                int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle error {rc}: {ERRORS.get(rc, 'unknown')}")
        return (out, w) if weights else out
    if weights:
        w = np.empty((B, H, Sq, Skv), dtype=np.float64)
        rc = lib.oracle_attn_fwd_weights_gqa(q.ctypes.data, k.ctypes.data, v.ctypes.data, code,
                                             out.ctypes.data, w.ctypes.data, B, H, Hkv, Sq, Skv,
                                             d, dv, float(scale), int(bool(causal)), lens_ptr,
                                             int(nthreads))
    else:
        rc = lib.oracle_attn_fwd_gqa(q.ctypes.data, k.ctypes.data, v.ctypes.data, code,
                                     out.ctypes.data, B, H, Hkv, Sq, Skv, d, dv, float(scale),
                                     int(bool(causal)), lens_ptr, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {ERRORS.get(rc, 'unknown')}")
    return (out, w) if weights else out
