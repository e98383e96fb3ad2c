"""The C-ABI library on the host: it loads, exports every declared entry
point, and its argument checks and kernel choice behave as documented.
No compute call is made (none of these reach a HIP API)."""
import ast
import ctypes
import math
import os
import re

import numpy as np
import pytest

import transformer_scaled_dot_attn_amd as attn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "attn.h")

A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
F32, BF16 = attn.F32, attn.BF16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    assert "attn_fwd" in names and "attn_fwd_ws" in names and len(names) >= 10, names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(attn.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_and_status_strings():
    assert attn.abi_version() == attn.ABI_VERSION
    for s in range(11):
        assert attn.status_string(s) and attn.status_string(s) != "unknown status"
    assert attn.status_string(99) == "unknown status"


def test_prefill_plan():
    """Launch plans of the measured workloads (no GPU call)."""
    assert attn.prefill_plan(1, 32, 4096, 4096, 128) == (1, 256, 1)   # prefill4096
    assert attn.prefill_plan(8, 32, 2048, 2048, 128) == (1, 256, 1)   # padded2048
    assert attn.prefill_plan(4, 12, 512, 512, 64) == (1, 128, 2)      # mha768
    assert attn.prefill_plan(4, 12, 512, 512, 64, masked=True) == (1, 128, 1)
    assert attn.prefill_plan(4, 12, 512, 512, 64, general=True) == (1, 128, 1)
    assert attn.prefill_plan(1, 32, 1024, 1024, 128) == (1, 128, 2)
    assert attn.prefill_plan(1, 32, 512, 512, 128) == (1, 64, 2)
    assert attn.prefill_plan(1, 32, 256, 256, 128) == (1, 64, 1)      # 4 key tiles: one group
    assert attn.prefill_plan(1, 32, 2048, 2048, 128) == (1, 128, 2)   # 256 blocks of 256 rows
    assert attn.prefill_plan(1, 32, 2048, 2048, 128, masked=True) == (1, 256, 1)
    assert attn.prefill_plan(2, 32, 2048, 2048, 128) == (1, 256, 1)   # 512 blocks
    assert attn.prefill_plan(1, 32, 512, 4096, 128) == (4, 256, 1)    # chunk: key-range splits
    with pytest.raises(attn.AttnError) as e:
        attn.prefill_plan(1, 32, 1, 4096, 128)                          # decode
    assert e.value.status == attn.E_UNSUPPORTED
    with pytest.raises(attn.AttnError) as e:
        attn.prefill_plan(1, 32, 64, 64, 96)
    assert e.value.status == attn.E_UNSUPPORTED
    with pytest.raises(attn.AttnError) as e:
        attn.prefill_plan(1, 32, 65, 64, 128)                           # Sq > Skv
    assert e.value.status == attn.E_SHAPE


def test_prefill_plan_properties():
    """Over random shapes: rows per block in {64, 128, 256}; key-range splits
    only with 256-row blocks and one key group; two key groups only without a
    mask or general logits, on blocks under 256 rows, with at least 8 key
    tiles; a mask or general logits never change the splits."""
    rng = np.random.default_rng(5)
    for _ in range(3000):
        B = int(rng.integers(1, 65))
        H = int(rng.choice([1, 2, 4, 8, 12, 16, 32, 64]))
        Skv = int(rng.integers(2, 70000))
        Sq = int(rng.integers(2, min(Skv, 9000) + 1))
        d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        masked, general = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        ns, bm, kg = attn.prefill_plan(B, H, Sq, Skv, d, dv, masked=masked, general=general)
        assert bm in (64, 128, 256) and kg in (1, 2) and 1 <= ns <= 16, (ns, bm, kg)
        if ns > 1:
            assert bm == 256 and kg == 1
        if kg == 2:
            assert not masked and not general and bm < 256 and (Skv + 63) // 64 >= 8
        assert attn.prefill_plan(B, H, Sq, Skv, d, dv)[0] == ns


def test_no_hip_error_recorded_before_a_launch_failure():
    assert attn.last_hip_error() == (0, "hipSuccess")


def test_library_shares_torchs_hip_runtime():
    """Loading the library before torch must not map a second HIP runtime:
    the library binds to the one torch carries, whatever the import order."""
    import subprocess
    import sys
    code = ("import transformer_scaled_dot_attn_amd as a; a.library(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') "
            "if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    maps = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(maps) == 1, maps


def v(B=1, H=1, Sq=4, Skv=4, d=64, scale=0.125, causal=1, dtype=BF16, q=A, k=A, vv=A, out=A):
    return attn.validate(q, k, vv, out, B, H, Sq, Skv, d, scale, causal, dtype)


def test_validate_accepts_supported_requests():
    assert v() == attn.OK
    assert v(d=128) == attn.OK
    assert v(Sq=1, Skv=8192, d=128) == attn.OK
    assert v(dtype=F32, d=16) == attn.OK
    assert v(dtype=F32, d=1, Sq=1, Skv=1) == attn.OK
    assert v(dtype=F32, d=128, Sq=3, Skv=7) == attn.OK
    # any finite scale: a scale that is not positive runs the general kernels
    assert v(scale=0.0) == attn.OK and v(scale=-0.125) == attn.OK
    assert v(scale=-0.125, Sq=1, Skv=100) == attn.OK and v(scale=-1.0, dtype=F32, d=16) == attn.OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), attn.E_NULL), (dict(k=0), attn.E_NULL), (dict(vv=0), attn.E_NULL),
    (dict(out=0), attn.E_NULL),
    (dict(dtype=2), attn.E_DTYPE), (dict(dtype=-1), attn.E_DTYPE),
    (dict(B=0), attn.E_SHAPE), (dict(H=-1), attn.E_SHAPE), (dict(Sq=0), attn.E_SHAPE),
    (dict(Skv=0), attn.E_SHAPE), (dict(d=0), attn.E_SHAPE), (dict(Sq=5, Skv=4), attn.E_SHAPE),
    (dict(B=1 << 20, H=1 << 10, Sq=1, Skv=1 << 16, d=128), attn.E_SHAPE),
    (dict(scale=float("inf")), attn.E_ARG), (dict(scale=float("nan")), attn.E_ARG),
    (dict(q=A + 8), attn.E_ALIGN), (dict(out=A + 2), attn.E_ALIGN),
    (dict(d=32), attn.E_UNSUPPORTED), (dict(d=96), attn.E_UNSUPPORTED),
    (dict(d=256), attn.E_UNSUPPORTED), (dict(dtype=F32, d=129), attn.E_UNSUPPORTED),
])
def test_validate_rejects(kw, code):
    assert v(**kw) == code


def test_bf16_head_rows_under_4gib():
    """The bf16 kernels address a head's K/V rows with 32-bit byte offsets:
    Skv * max(d, d_v) * 2 must stay below 2^32."""
    assert v(Sq=2, Skv=(1 << 24) - 1, d=128) == attn.OK
    assert v(Sq=2, Skv=1 << 24, d=128) == attn.E_UNSUPPORTED
    assert v(Sq=1, Skv=1 << 24, d=128) == attn.E_UNSUPPORTED
    assert v(Sq=2, Skv=1 << 24, d=64) == attn.OK
    assert vm(mask=None, dtype=BF16, Sq=2, Skv=1 << 24, d=64, dv=128) == attn.E_UNSUPPORTED
    assert v(dtype=F32, Sq=2, Skv=1 << 24, d=128) == attn.OK


def test_check_order_null_before_shape():
    assert v(q=0, B=0) == attn.E_NULL
    assert v(B=0, scale=float("nan")) == attn.E_SHAPE


def test_kernel_choice():
    assert attn.kernel_for(4096, 4096, 128, BF16) == "prefill_bf16_mfma"
    assert attn.kernel_for(512, 512, 64, BF16) == "prefill_bf16_mfma"
    assert attn.kernel_for(2, 9, 64, BF16) == "prefill_bf16_mfma"
    assert attn.kernel_for(1, 8192, 128, BF16) == "decode_bf16_stream"
    assert attn.kernel_for(64, 64, 16, F32) == "generic_f32"
    assert attn.kernel_for(1, 64, 16, F32) == "generic_f32"
    assert attn.kernel_for(4, 4, 48, BF16) is None
    assert attn.kernel_for(5, 4, 64, BF16) is None


def _stream_rows(B, H, Hkv, Skv, d):
    """Partial rows of the stream decode: one slot per (wave, pair) segment,
    at most (2048 waves at d = 128, 4096 at d = 64, and no more than tiles)
    + pairs slots, of min(32, H / H_kv) head rows each."""
    group = H // Hkv
    pairs = B * Hkv * ((group + 31) // 32)
    waves = min(2048 if d == 128 else 4096, max(1, pairs * ((Skv + 31) // 32)))
    return (waves + pairs) * min(32, group), pairs


def test_workspace_sizes():
    # decode needs (m, l, acc[d]) partials and two wave indices per pair;
    # the other kernels need none here
    assert attn.workspace_bytes(1, 32, 4096, 4096, 128, BF16) == 0
    assert attn.workspace_bytes(1, 1, 64, 64, 16, F32) == 0
    w = attn.workspace_bytes(64, 32, 1, 8192, 128, BF16)
    rows, pairs = _stream_rows(64, 32, 32, 8192, 128)
    assert w >= rows * (128 + 2) * 4 + pairs * 2 * 4
    assert w <= rows * (128 + 2) * 4 + pairs * 2 * 4 + 3 * 256
    assert w % 256 == 0
    # a short problem needs few slots
    small = attn.workspace_bytes(1, 4, 1, 40, 64, BF16)
    rows, pairs = _stream_rows(1, 4, 4, 40, 64)
    assert rows == 8 + 4 and small <= 3 * 256 + rows * 66 * 4
    assert attn.workspace_bytes(0, 32, 1, 8192, 128, BF16) == 0


def vg(B=2, H=8, Hkv=2, Sq=4, Skv=4, d=64, scale=0.125, causal=1, dtype=BF16):
    return attn.library().attn_validate_gqa(A, A, A, A, B, H, Hkv, Sq, Skv, d, scale, causal,
                                            dtype)


def test_validate_gqa():
    # H_kv must divide H; H_kv = H is the multi-head case
    for Hkv in (1, 2, 4, 8):
        assert vg(Hkv=Hkv) == attn.OK
        assert vg(Hkv=Hkv, Sq=1, Skv=100, d=128) == attn.OK
        assert vg(Hkv=Hkv, dtype=F32, d=20) == attn.OK
    for Hkv in (0, -2, 3, 5, 16):
        assert vg(Hkv=Hkv) == attn.E_SHAPE, Hkv
    assert vg(Hkv=2, d=32) == attn.E_UNSUPPORTED
    assert vg(H=6, Hkv=3) == attn.OK and vg(H=6, Hkv=4) == attn.E_SHAPE


def test_gqa_workspace_sizes():
    lib = attn.library()
    # one partial per (wave, pair) segment, min(32, H / H_kv) head rows each
    for Hkv in (1, 8, 32):
        w = lib.attn_workspace_bytes_gqa(64, 32, Hkv, 1, 8192, 128, BF16)
        rows, pairs = _stream_rows(64, 32, Hkv, 8192, 128)
        assert rows * (128 + 2) * 4 + pairs * 8 <= w <= rows * (128 + 2) * 4 + pairs * 8 + 768
        assert w % 256 == 0
        assert attn.workspace_bytes(64, 32, 1, 8192, 128, BF16, kv_heads=Hkv) == w
    assert lib.attn_workspace_bytes_gqa(64, 32, 32, 1, 8192, 128, BF16) == \
        attn.workspace_bytes(64, 32, 1, 8192, 128, BF16)
    assert lib.attn_workspace_bytes_gqa(64, 32, 5, 1, 8192, 128, BF16) == 0
    assert lib.attn_workspace_bytes_gqa(2, 32, 8, 4096, 4096, 128, BF16) == 0


def test_prefill_split_workspace():
    # a grid of at least 2 blocks per CU needs no splits and no workspace
    assert attn.workspace_bytes(1, 32, 4096, 4096, 128, BF16) == 0
    assert attn.workspace_bytes(4, 32, 1024, 1024, 128, BF16) == 0
    # a short query chunk against a long cache splits the key range: one
    # (m, l, acc[d]) partial per query row and split
    w = attn.workspace_bytes(1, 32, 512, 4096, 128, BF16)
    assert w >= 1 * 32 * 512 * 2 * (128 + 2) * 4 and w % 256 == 0
    assert attn.workspace_bytes(1, 32, 256, 8192, 64, BF16, kv_heads=8) > 0
    # at most 16 splits, each of at least 8 key tiles
    assert attn.workspace_bytes(1, 1, 2, 64, 128, BF16) == 0
    assert attn.workspace_bytes(1, 1, 2, 100000, 128, BF16) <= 16 * 2 * (128 + 2) * 4 + 512


def test_profile_names():
    names = attn.profile_names()
    assert names == ["prefill_bf16_mfma", "decode_bf16_partial", "decode_bf16_combine",
                     "generic_f32", "prefill_bf16_combine", "prefill_mask_tiles",
                     "decode_mask_tiles"]


def test_python_layer_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="GPU device"):
        attn.fwd(q, q, q)
    with pytest.raises(ValueError, match="4-D"):
        attn.fwd(q[0], q, q)
    with pytest.raises(ValueError):
        attn.fwd(q.to(torch.float16), q, q)
    q3 = torch.zeros(1, 3, 4, 64)
    k2 = torch.zeros(1, 2, 4, 64)
    with pytest.raises(ValueError):
        attn.fwd(q3, k2, k2)


def vm(mask=A, sb=0, sh=0, si=0, B=2, H=4, Hkv=2, Sq=8, Skv=64, d=128, dtype=BF16, scale=0.125,
       dv=None):
    return attn.validate_ex(A, A, A, A, B, H, Hkv, Sq, Skv, d, d if dv is None else dv, scale, 1,
                            mask, sb, sh, si, dtype)


def test_validate_mask():
    # NULL mask: the attn_validate_gqa checks alone
    assert vm(mask=None) == attn.OK
    assert vm(sb=4 * 8 * 64, sh=8 * 64, si=64) == attn.OK          # dense [B,H,Sq,Skv]
    assert vm(sb=8 * 64, sh=0, si=64) == attn.OK                    # [B,1,Sq,Skv]
    assert vm(sb=64, sh=0, si=0) == attn.OK                         # key padding [B,1,1,Skv]
    assert vm(Sq=1, sb=68, sh=0, si=0, Skv=65) == attn.OK           # padded rows
    assert vm(dtype=F32, d=40, si=64) == attn.OK
    # word-aligned base and strides
    assert vm(mask=A + 2) == attn.E_ALIGN
    assert vm(si=65) == attn.E_ALIGN
    assert vm(sb=66) == attn.E_ALIGN
    assert vm(sh=6) == attn.E_ALIGN
    # negative strides, overflowing extents
    assert vm(si=-64) == attn.E_SHAPE
    assert vm(sb=-4) == attn.E_SHAPE
    assert vm(B=2, sb=1 << 62) == attn.E_SHAPE
    assert vm(si=1 << 27) == attn.E_UNSUPPORTED and vm(si=(1 << 27) - 64) == attn.OK
    # the shared checks come first
    assert vm(B=0, mask=A + 1) == attn.E_SHAPE
    assert vm(scale=float("nan")) == attn.E_ARG
    assert vm(Hkv=3) == attn.E_SHAPE


def test_validate_value_width():
    # d_v != d: fp32 d_v in 1..128
    assert vm(mask=None, dtype=F32, d=4, dv=2) == attn.OK
    assert vm(mask=None, dtype=F32, d=128, dv=16) == attn.OK
    assert vm(mask=None, dtype=F32, d=20, dv=128) == attn.OK
    assert vm(mask=None, dtype=F32, d=20, dv=129) == attn.E_UNSUPPORTED
    assert vm(mask=None, dtype=F32, d=20, dv=0) == attn.E_SHAPE
    # bf16: d and d_v each in {64, 128}
    assert vm(mask=None, dtype=BF16, d=128, dv=64) == attn.OK
    assert vm(mask=None, dtype=BF16, d=64, dv=128) == attn.OK
    assert vm(mask=None, dtype=BF16, d=64, dv=32) == attn.E_UNSUPPORTED
    assert vm(mask=None, dtype=BF16, d=128, dv=96) == attn.E_UNSUPPORTED
    assert vm(mask=None, dtype=BF16, d=64, dv=64) == attn.OK
    assert vm(mask=None, dtype=BF16, Sq=1, d=128, dv=128) == attn.OK


def test_masked_prefill_workspace():
    # key-tile marks: one byte per (batch, query tile, key tile), after any split partials
    base = attn.workspace_bytes(2, 32, 4096, 4096, 128, BF16)
    masked = attn.workspace_bytes(2, 32, 4096, 4096, 128, BF16, masked=True)
    assert base == 0 and masked >= 2 * 16 * 64 and masked % 256 == 0
    split = attn.workspace_bytes(1, 2, 300, 8000, 128, BF16)
    assert split > 0
    assert attn.workspace_bytes(1, 2, 300, 8000, 128, BF16, masked=True) >= split + 2 * 125
    # decode: a visible-tile count and a list of up to ceil(Skv / 32) tiles per pair
    dec = attn.workspace_bytes(4, 8, 1, 5000, 128, BF16)
    dec_m = attn.workspace_bytes(4, 8, 1, 5000, 128, BF16, masked=True)
    assert dec_m - dec >= 32 * 4 + 32 * 157 * 4 and dec_m - dec <= 32 * 4 + 32 * 157 * 4 + 512
    # fp32: a mask needs nothing
    assert attn.workspace_bytes(1, 2, 64, 64, 32, F32, masked=True) == 0
    # beyond the list size the marks are not used
    assert attn.workspace_bytes(1, 1, 64, 200000, 128, BF16, masked=True) == \
        attn.workspace_bytes(1, 1, 64, 200000, 128, BF16)


def test_noalloc_refuses_problems_beyond_the_scratch_array():
    """attn_fwd_noalloc checks the problem's temporary memory against its
    fixed scratch array on the host, before any HIP call: a decode whose
    partials exceed the array is refused with ATTN_E_SCRATCH."""
    lib = attn.library()
    cap = attn.noalloc_scratch_bytes()
    assert cap == 64 << 20
    B, H, Hkv, Skv, d = 4096, 32, 1, 8192, 128
    assert attn.workspace_bytes(B, H, 1, Skv, d, BF16, kv_heads=Hkv) > cap
    rc = lib.attn_fwd_noalloc(A, A, A, A, B, H, Hkv, 1, Skv, d, d, ctypes.c_float(0.088), 0,
                              None, None, 0, 0, 0, BF16, None)
    assert rc == attn.E_SCRATCH, attn.status_string(rc)
    # the argument checks of attn_fwd_ex come first
    rc = lib.attn_fwd_noalloc(A, A, A, None, B, H, Hkv, 1, Skv, d, d, ctypes.c_float(0.088), 0,
                              None, None, 0, 0, 0, BF16, None)
    assert rc == attn.E_NULL
    rc = lib.attn_fwd_noalloc(A, A, A, A, B, H, 3, 1, Skv, d, d, ctypes.c_float(0.088), 0,
                              None, None, 0, 0, 0, BF16, None)
    assert rc == attn.E_SHAPE


def vb(bias=A, bsb=0, bsh=0, bsi=0, B=2, H=4, Hkv=2, Sq=8, Skv=64, d=128, dtype=BF16, mask=None,
       msi=0):
    return attn.library().attn_validate_bias(A, A, A, A, B, H, Hkv, Sq, Skv, d, d, 0.125, 1, mask,
                                             0, 0, msi, bias, bsb, bsh, bsi, dtype)


def test_validate_bias():
    """Additive-bias layout checks: 16-byte base, strides >= 0 and multiples
    of 4 elements, 32-bit row offsets for a wave's rows; a NULL bias is the
    attn_validate_ex checks alone."""
    assert vb(bias=None) == attn.OK
    assert vb(bsb=4 * 8 * 64, bsh=8 * 64, bsi=64) == attn.OK       # dense [B,H,Sq,Skv]
    assert vb(bsb=64) == attn.OK                                    # [B,1,1,Skv]
    assert vb(Sq=1, Skv=65, bsb=68) == attn.OK                      # padded rows
    assert vb(dtype=F32, d=16, bsi=64) == attn.OK
    assert vb(bias=A + 8) == attn.E_ALIGN
    assert vb(bsi=66) == attn.E_ALIGN and vb(bsh=2) == attn.E_ALIGN and vb(bsb=1) == attn.E_ALIGN
    assert vb(bsi=-64) == attn.E_SHAPE and vb(bsh=-4) == attn.E_SHAPE
    assert vb(B=2, bsb=1 << 62) == attn.E_SHAPE
    # bf16 rows of 2 bytes: 32 rows of stride si must stay below 2^32 bytes
    assert vb(bsi=1 << 26) == attn.E_UNSUPPORTED and vb(bsi=(1 << 26) - 64) == attn.OK
    assert vb(dtype=F32, d=16, bsi=1 << 25) == attn.E_UNSUPPORTED
    # the mask checks come first
    assert vb(mask=A + 2, bias=A + 8) == attn.E_ALIGN
    assert vb(mask=A, msi=65) == attn.E_ALIGN
