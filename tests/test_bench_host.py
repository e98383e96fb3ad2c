"""Host-side bookkeeping of bench.py, run on the CPU with the kernel launches
and their timing replaced by stubs: the masked-run rows (visible-pair flops,
visible K/V-row bytes) and the grouped-decode rows are assembled without a
GPU, so an error there shows up before a GPU run."""
import math
import types

import numpy as np

import bench
import workloads as W


class _Attn:
    BF16 = 1
    masked = False

    def fwd(self, *a, **kw):
        _Attn.masked = kw.get("mask") is not None


def _stub_timing(monkeypatch):
    calls = []

    def timed(attn, fn, steps, warmup, kernels):
        fn()
        calls.append(kernels)
        # the mask pre-passes are absent from an unmasked call, as on the GPU
        res = {}
        for k in kernels:
            ran = not (k.endswith("_mask_tiles") and not _Attn.masked)
            res[k] = {"ms": 1.0 if ran else math.nan, "median_us": 900.0 if ran else None,
                      "min_us": 800.0 if ran else None, "n": 3 if ran else 0}
        return res

    def rounds(attn, fns, steps, warmup, kernels, rounds=5):
        return [timed(attn, fn, steps, warmup, kernels) for fn in fns]

    monkeypatch.setattr(bench, "timed_calls", timed)
    monkeypatch.setattr(bench, "timed_rounds", rounds)
    return calls


def _host_workloads():
    # mask_to_torch and bias_to_torch would upload; the bookkeeping only needs the array
    names = {k: getattr(W, k) for k in dir(W) if not k.startswith("__")}
    names["mask_to_torch"] = lambda m, device="cuda": m
    names["bias_to_torch"] = lambda b, device="cuda": b
    return types.SimpleNamespace(**names)


def _inputs(w):
    lens = W.kv_lens_for(w)
    return {"q": None, "k": None, "v": None, "scale": 1.0 / math.sqrt(w.d),
            "kv_lens": None if lens is None else np.asarray(lens, dtype=np.int32),
            "kv_lens_host": None if lens is None else [int(x) for x in lens], "sha256": "0" * 64}


def test_mask_rows(monkeypatch):
    calls = _stub_timing(monkeypatch)
    runs = []
    for kind, name in (("prefill", "prefill4096_bf16"), ("decode", "decode8192_bf16"),
                       ("decode", "gqa_decode8192_bf16")):
        w = W.WORKLOADS[name]
        runs.append((kind, w, _inputs(w), None))
    rows = bench.mask_runs(_Attn(), _host_workloads(), runs, steps=1, warmup=0)
    assert len(rows) == 9 + 3 + 3 and len(calls) == len(rows)
    for r in rows:
        assert r["ms_per_call"] > 0 and math.isfinite(r["time_vs_unmasked"])
    pre = [r for r in rows if r["workload"] == "prefill4096_bf16"]
    assert pre[0]["mask"] == "none" and pre[0]["visible_pairs_share"] == 1.0
    assert pre[1]["visible_pairs_share"] == 1.0 and pre[2]["visible_pairs_share"] == 1.0
    for r in pre[3:7]:
        assert 0.0 < r["visible_pairs_share"] < 1.0 and r["TFLOP/s"] > 0
    # the two additive biases (finite values) hide no pair
    assert [r["mask"].split()[0] for r in pre[7:]] == ["bias", "bias"]
    for r in pre[7:]:
        assert r["visible_pairs_share"] == 1.0
    # documents of 512 and a window of 256 open about an eighth of the causal pairs
    assert 0.10 < pre[5]["visible_pairs_share"] < 0.15
    assert 0.10 < pre[6]["visible_pairs_share"] < 0.15
    for name in ("decode8192_bf16", "gqa_decode8192_bf16"):
        dec = [r for r in rows if r["workload"] == name]
        assert "visible_kv_rows_share" not in dec[0]
        # the left half of every sequence hidden: about half of the rows
        assert 0.45 < dec[1]["visible_kv_rows_share"] < 0.55
        assert dec[1]["GB/s"] < dec[0]["GB/s"]
        # random [B,H,1,S] masks: a K/V row is seen if any query head of its group sees it
        g = W.WORKLOADS[name].H // W.WORKLOADS[name].kv_heads
        assert abs(dec[2]["visible_kv_rows_share"] - (1.0 - 0.5 ** g)) < 0.02


def test_grouped_decode_rows(monkeypatch):
    _stub_timing(monkeypatch)
    w = W.WORKLOADS["decode8192_bf16"]
    have = {w.name: _inputs(w)}
    import torch
    monkeypatch.setattr(W, "device_inputs", lambda w, dev="cuda", **kw: _inputs(w))
    monkeypatch.setattr(torch, "empty_like", lambda x: None)
    rows = bench.gqa_decode_sweep(_Attn(), W, "cpu", 1, 0, have=have)
    by = {r["H_kv"]: r for r in rows}
    assert set(by) >= {32, 8, 1}
    for hkv, r in by.items():
        assert abs(r["intensity_flop_per_byte"] - 32 / hkv) < 0.05 * 32 / hkv
        assert r["roofline"]["bound"] == "hbm" and r["roofline"]["frac"] > 0


def test_prefill_config_rows(monkeypatch):
    _stub_timing(monkeypatch)
    import torch
    monkeypatch.setattr(W, "device_inputs", lambda w, dev="cuda", **kw: _inputs(w))
    monkeypatch.setattr(torch, "empty_like", lambda x: None)
    rows = bench.prefill_configs(_Attn(), W, "cpu", 1, 0)
    by = {r["workload"]: r for r in rows}
    # C2: 4 d flops per causal pair of 4 x 12 sequences of 512
    assert by["mha768_bf16"]["flop_per_call"] == 4 * 64 * 48 * 512 * 513 / 2
    # C4: the drawn lengths set the visible pairs, below the unpadded count
    pad = by["padded2048_bf16"]
    full = 4 * 128 * 8 * 32 * 2048 * 2049 / 2
    assert 0.2 * full < pad["flop_per_call"] < full
    for r in rows:
        # the stub times the prefill and the split-combine kernel at 1 ms each
        assert r["ms_per_call"] == 2.0 and r["frac"] == r["TFLOP/s"] / bench.PEAK_BF16_TFLOPS
        assert r["median_us"] == 1800.0 and r["min_us"] == 1600.0 and len(r["sha256"]) == 64


def test_sweep_slopes():
    # time growing as S^2 from S = 1024 on gives exponents of 2 and a fit of 2
    rows = [{"S": S, "ms_per_call": 0.01 * max(1.0, (S / 1024) ** 2)}
            for S in (128, 256, 512, 1024, 2048, 4096, 8192)]
    sl = bench.sweep_slopes(rows)
    assert [round(x["exponent"], 6) for x in sl["per_doubling"]] == [0, 0, 0, 2, 2, 2]
    assert abs(sl["fit_S_ge_1024"] - 2.0) < 1e-12


def test_cpu_baseline_rows(monkeypatch):
    """Every configuration gets an oracle row: GFLOP/s for prefill (visible
    pairs of the timed slices), GB/s for decode (their K/V rows, q, out,
    lengths); the oracle itself is stubbed here."""
    import oracle
    seen = []
    monkeypatch.setattr(oracle, "attention",
                        lambda q, k, v, scale, causal, lens, nthreads=0: seen.append(q.shape))
    res = bench.cpu_baseline(4)
    rows = {r["workload"]: r for r in res["configs"]}
    assert set(rows) == {"tiny_f32", "mha768_bf16", "prefill4096_bf16", "padded2048_bf16",
                         "decode8192_bf16"}
    assert seen[2] == (1, 32, 4096, 128) and seen[3][:2] == (32, 1) and seen[4][:2] == (128, 1)
    for name, r in rows.items():
        assert r["seconds"] > 0 and r["threads"] <= 4
        assert ("GB/s" in r) == (name == "decode8192_bf16")
    assert res["unit"] == "TFLOP/s" and res["nproc"] >= 1 and res["cores"] == 4
    assert res["value"] == rows["prefill4096_bf16"]["GFLOP/s"] / 1e3



def test_code_digest_ignores_comments_only():
    """The digest that ties a profile's counters to the kernel code: comment
    and blank-line edits keep it, any change to the code changes it, and
    comment markers inside literals are code."""
    a = 'int f(int x) {  // twice\n    /* no */ return 2 * x;\n}\nconst char* s = "a // b";\n'
    b = '// header\nint f(int x) {\n\n    return 2 * x;   \n}\nconst char* s = "a // b";\n'
    c = 'int f(int x) {\n    return 3 * x;\n}\nconst char* s = "a // b";\n'
    d = 'int f(int x) {\n    return 2 * x;\n}\nconst char* s = "a ";\n'
    assert bench.strip_comments(a) == bench.strip_comments(b)
    assert bench.strip_comments(a) != bench.strip_comments(c)
    assert bench.strip_comments(a) != bench.strip_comments(d)
    assert bench.strip_comments("x = '\"'; // q\ny = 1;") == "x = '\"';\ny = 1;"


def test_committed_profiles_match_the_kernel_code():
    """Every committed summary carries the digest of the code it measured;
    bench reports its traffic only while that digest matches."""
    import os
    prof = os.path.join(bench.ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.endswith(".md") and "__" in f]
    assert names
    for f in names:
        kernel, workload = f[:-3].split("__")
        assert bench.profiled_traffic(kernel, workload) is not None, f
