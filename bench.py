#!/usr/bin/env python3
"""Attention forward throughput on one MI355X.

One step is one pass of the whole path: a causal prefill over
B=1, H=32, S=4096, d=128 (d_model 4096) and a split-KV decode over
B=64, H=32, one query against KV caches of capacity 8192 with valid lengths
drawn uniformly from [512, 8192], all bf16 with fp32 accumulation, inputs
resident in HBM before timing starts.

Printed (one JSON line): prefill TFLOP/s as `value` (algorithmic flops: 4*d
per visible (query, key) pair), decode KV-read GB/s under `decode` (bytes of
the valid K and V rows plus q, out and the lengths), each with a roofline
entry for its dominant kernel computed from that kernel's own HIP-event
durations, and the float64 CPU oracle timed on a bounded sample of the same
workload as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

COPY_BYTES = 1 << 30        # calibration copy size

PREFILL = "prefill4096_bf16"
DECODE = "decode8192_bf16"


def prefill_flops(w, lens=None) -> float:
    """4*d flops per visible (query, key) pair; padded rows and masked pairs
    are not counted."""
    total = 0
    for b in range(w.B):
        L = w.Skv if lens is None else int(min(max(int(lens[b]), 0), w.Skv))
        n = min(w.Sq, L)
        off = L - n
        if w.causal:
            # query i (absolute position off+i) sees off+i+1 keys
            pairs = n * (off + 1) + n * (n - 1) // 2
        else:
            pairs = n * L
        total += pairs
    return 4.0 * w.d * w.H * total


def decode_bytes(w, lens) -> float:
    """Bytes the decode must move: valid K and V rows (of the K/V heads),
    q, out, kv_lens."""
    kv = 2 * 2 * w.d * w.kv_heads * int(sum(int(min(max(int(x), 0), w.Skv)) for x in lens))
    qo = 2 * (2 * w.B * w.H * w.d)
    return float(kv + qo + 4 * w.B)


def decode_flops(w, lens) -> float:
    """4*d flops per (query head, valid key) pair."""
    return 4.0 * w.d * w.H * float(sum(int(min(max(int(x), 0), w.Skv)) for x in lens))


def kernel_stats(attn, kernels):
    """Per-launch HIP-event durations of the named library kernels since the
    last profile reset: {name: {"ms": mean, "median_us", "min_us", "n"}}
    (ms is NaN for a kernel that did not run)."""
    res = {}
    for k in kernels:
        t = attn.profile_samples(k)
        if t:
            res[k] = {"ms": sum(t) / len(t), "median_us": 1e3 * statistics.median(t),
                      "min_us": 1e3 * min(t), "n": len(t)}
        else:
            res[k] = {"ms": float("nan"), "median_us": None, "min_us": None, "n": 0}
    return res


def timed_calls(attn, fn, steps, warmup, kernels):
    """Run fn warmup + steps times; per-launch statistics of each named
    library kernel over the timed calls (see kernel_stats)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    attn.profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    st = kernel_stats(attn, kernels)
    attn.profile_enable(False)
    return st


def timed_rounds(attn, fns, steps, warmup, kernels, rounds=5):
    """As timed_calls for several callables, interleaved: after warming all
    up, each of `rounds` rounds runs every callable steps / rounds times in
    turn, so they share one clock and power history (a row measured first
    would otherwise sit in the power transient of a cold start).  Returns
    one kernel_stats-like dict per callable."""
    import torch
    for fn in fns:
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    per = max(1, steps // rounds)
    samples = [{k: [] for k in kernels} for _ in fns]
    for _ in range(rounds):
        for i, fn in enumerate(fns):
            attn.profile_enable(True)
            for _ in range(per):
                fn()
            torch.cuda.synchronize()
            for k in kernels:
                samples[i][k] += attn.profile_samples(k)
            attn.profile_enable(False)
    out = []
    for smp in samples:
        res = {}
        for k, t in smp.items():
            if t:
                res[k] = {"ms": sum(t) / len(t), "median_us": 1e3 * statistics.median(t),
                          "min_us": 1e3 * min(t), "n": len(t)}
            else:
                res[k] = {"ms": float("nan"), "median_us": None, "min_us": None, "n": 0}
        out.append(res)
    return out


def op_stats(st, kernels):
    """Mean ms of one call made of the named kernels (those that ran), and the
    median and min of the per-call sums."""
    ran = [k for k in kernels if st[k]["n"]]
    ms = sum(st[k]["ms"] for k in ran)
    return ms, sum(st[k]["median_us"] for k in ran), sum(st[k]["min_us"] for k in ran)


def gqa_decode_sweep(attn, W, dev, steps, warmup,
                     names=("decode8192_bf16", "gqa_decode8192_bf16", "mqa_decode8192_bf16"),
                     have=None):
    """Decode at 32, 8 and 1 K/V heads for 32 query heads ("Attention from
    First Principles", section 10, exercise F): bytes moved fall by H / H_kv
    while the flops stay, so the intensity is H / H_kv.  `have` maps workload
    names to device inputs already drawn (the step's), which are reused."""
    import torch
    rows = []
    have = have or {}
    for name in names:
        w = W.WORKLOADS[name]
        x = have[name] if name in have else W.device_inputs(w, dev, digest=True)
        out = torch.empty_like(x["q"])
        fn = lambda: attn.fwd(x["q"], x["k"], x["v"], out, causal=w.causal,
                              kv_lens=x["kv_lens"], scale=x["scale"])
        kern = ("decode_bf16_partial", "decode_bf16_combine")
        t = timed_calls(attn, fn, steps, warmup, kern)
        ms, med, mn = op_stats(t, kern)
        lens = x["kv_lens_host"]
        nbytes, flops = decode_bytes(w, lens), decode_flops(w, lens)
        p_ms = t["decode_bf16_partial"]["ms"]
        kv_bytes = nbytes - 2 * 2 * w.B * w.H * w.d  # what the partial kernel reads
        kernel = "decode_bf16_partial"  # the stream kernel, at every K/V head count
        rows.append({"workload": name, "H": w.H, "H_kv": w.kv_heads, "ms_per_call": ms,
                     "median_us": med, "min_us": mn, "sha256": x.get("sha256"),
                     "GB/s": nbytes / (ms * 1e-3) / 1e9, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                     "intensity_flop_per_byte": flops / nbytes,
                     "roofline": {"kernel": kernel, "bound": "hbm",
                                  "achieved": kv_bytes / (p_ms * 1e-3) / 1e9,
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": kv_bytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                  "traffic": profiled_traffic(kernel, name),
                                  "algorithmic_bytes_per_launch": kv_bytes,
                                  "avg_launch_ms": p_ms}})
        del x, out
        torch.cuda.empty_cache()
    return rows


def prefill_sweep(attn, W, dev, steps, warmup):
    """Causal prefill, B=1, H=32, d=128, over S = 128 .. 8192: TFLOP/s by S
    ("Attention from First Principles", section 10, exercise D: work grows
    as S^2, so time should too once the GPU is full)."""
    import torch
    rows = []
    for S in (128, 256, 512, 1024, 2048, 4096, 8192):
        w = W.Workload(f"prefill{S}_sweep", 1, 32, S, S, 128, "bf16", True, 100 + S)
        x = W.device_inputs(w, dev)
        out = torch.empty_like(x["q"])
        fn = lambda: attn.fwd(x["q"], x["k"], x["v"], out, causal=True, scale=x["scale"])
        kern = ("prefill_bf16_mfma", "prefill_bf16_combine")
        t = timed_calls(attn, fn, steps, warmup, kern)
        ms, med, mn = op_stats(t, kern)  # the combine runs only with key splits
        flops = prefill_flops(w)
        rows.append({"S": S, "ms_per_call": ms, "median_us": med, "min_us": mn,
                     "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                     "key_splits": attn.workspace_bytes(1, 32, S, S, 128, attn.BF16) > 0})
        del x, out
        torch.cuda.empty_cache()
    return rows


def prefill_configs(attn, W, dev, steps, warmup,
                    names=("mha768_bf16", "padded2048_bf16", "gqa_prefill2048_bf16")):
    """The other bf16 prefill workloads (d_model 768 at S = 512; causal with
    right padding, lengths U[256, 2048]; grouped K/V heads at S = 2048),
    each timed on its own: TFLOP/s of 4*d flops per visible pair."""
    import torch
    rows = []
    for name in names:
        w = W.WORKLOADS[name]
        x = W.device_inputs(w, dev, digest=True)
        out = torch.empty_like(x["q"])
        fn = lambda: attn.fwd(x["q"], x["k"], x["v"], out, causal=w.causal,
                              kv_lens=x["kv_lens"], scale=x["scale"])
        kern = ("prefill_bf16_mfma", "prefill_bf16_combine")
        t = timed_calls(attn, fn, steps, warmup, kern)
        ms, med, mn = op_stats(t, kern)  # the combine runs only with key splits
        flops = prefill_flops(w, x["kv_lens_host"])
        tflops = flops / (ms * 1e-3) / 1e12
        rows.append({"workload": name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "S": w.Sq,
                     "d": w.d, "ms_per_call": ms, "median_us": med, "min_us": mn,
                     "sha256": x["sha256"], "TFLOP/s": tflops,
                     "frac": tflops / PEAK_BF16_TFLOPS, "flop_per_call": flops})
        del x, out
        torch.cuda.empty_cache()
    return rows


def mask_runs(attn, W, runs, steps, warmup):
    """The step's workloads again with explicit allowed-masks (True = may
    attend, ANDed with the causal and length rules; "Attention from Scratch",
    KubeDojo module 1.4.3, Part 3), and the prefill with an additive bias of
    finite values (the float mask of its Part 7; every pair stays visible),
    against the same call unmasked.  Prefill
    counts 4*d flops per visible (query, key) pair -- allowed by the mask and
    by the causal rule -- the algorithmic work; decode counts the bytes of the
    K/V rows some query head of their group may see, plus q, out and the mask."""
    import numpy as np
    import torch
    rows = []
    for kind, w, x, out in runs:
        if kind == "prefill":
            S = w.Skv
            masks = [("none", None),
                     ("all true [1,1,1,S]", np.ones((1, 1, 1, S), dtype=bool)),
                     ("all true [1,1,S,S]", np.ones((1, 1, w.Sq, S), dtype=bool)),
                     ("key padding [1,1,1,S], first 256 keys hidden",
                      W.key_padding_mask([256], [S], S)),
                     ("random [1,1,S,S], density 0.5", W.random_mask(5, (1, 1, w.Sq, S), 0.5)),
                     ("8 packed documents of 512 [1,1,S,S]", W.document_mask([S // 8] * 8)),
                     ("sliding window of 256 [1,1,S,S]", W.window_mask(S, 256))]
            biases = [("bias [1,1,S,S], N(0, 4) values", W.random_bias(8, (1, 1, w.Sq, S), "bf16")),
                      ("bias [1,H,1,S], N(0, 4) values", W.random_bias(9, (1, w.H, 1, S), "bf16"))]
            kernels = ("prefill_bf16_mfma", "prefill_mask_tiles")
        else:
            lens = x["kv_lens_host"]
            starts = np.asarray(lens) // 2
            masks = [("none", None),
                     ("left padding [B,1,1,Skv], first half of each sequence hidden",
                      W.key_padding_mask(starts, np.full(w.B, w.Skv), w.Skv)),
                     ("random [B,H,1,Skv], density 0.5",
                      W.random_mask(6, (w.B, w.H, 1, w.Skv), 0.5))]
            biases = []
            kernels = ("decode_bf16_partial", "decode_bf16_combine", "decode_mask_tiles")
        base = None
        tms = [None if m is None else W.mask_to_torch(m) for _, m in masks]
        tbs = [W.bias_to_torch(bb) for _, bb in biases]
        fns = [(lambda tm=tm: attn.fwd(x["q"], x["k"], x["v"], out, causal=w.causal,
                                       kv_lens=x["kv_lens"], scale=x["scale"], mask=tm))
               for tm in tms]
        fns += [(lambda tb=tb: attn.fwd(x["q"], x["k"], x["v"], out, causal=w.causal,
                                        kv_lens=x["kv_lens"], scale=x["scale"], bias=tb))
                for tb in tbs]
        # the masks and biases interleaved
        stats = timed_rounds(attn, fns, steps, warmup, kernels)
        # a bias hides no pair: its rows count as unmasked ones
        for (label, m), t in zip(masks + [(lb, None) for lb, _ in biases], stats):
            ms, med, mn = op_stats(t, kernels)  # kernels a call did not launch are left out
            base = ms if base is None else base
            row = {"workload": w.name, "mask": label, "ms_per_call": ms, "median_us": med,
                   "min_us": mn, "time_vs_unmasked": ms / base}
            if kind == "prefill":
                if m is None:
                    flops = prefill_flops(w, x["kv_lens_host"])
                else:  # the step's prefill has B = 1 and no lengths; masks here are [1,1,*,S]
                    rule = np.tril(np.ones((w.Sq, w.Skv), dtype=bool), w.Skv - w.Sq)
                    vis = np.broadcast_to(m[0, 0], (w.Sq, w.Skv)) & (rule if w.causal else True)
                    flops = 4.0 * w.d * w.H * w.B * float(np.count_nonzero(vis))
                row["visible_pairs_share"] = flops / prefill_flops(w, x["kv_lens_host"])
                row["TFLOP/s"] = flops / (ms * 1e-3) / 1e12
            else:
                nbytes = decode_bytes(w, x["kv_lens_host"])
                if m is not None:
                    # algorithmic bytes: the K/V rows some query head of the group may see
                    lens = np.asarray(x["kv_lens_host"])
                    seen = np.broadcast_to(m[:, :, 0, :], (w.B, w.H, w.Skv)) & \
                        (np.arange(w.Skv)[None, None, :] < lens[:, None, None])
                    kv_seen = seen.reshape(w.B, w.kv_heads, w.H // w.kv_heads, w.Skv).any(axis=2)
                    nbytes += 2 * 2 * w.d * float(np.count_nonzero(kv_seen)) \
                        - 2 * 2 * w.d * w.kv_heads * float(lens.clip(0, w.Skv).sum()) \
                        + int(np.prod(m.shape[:3])) * w.Skv
                    row["visible_kv_rows_share"] = float(np.count_nonzero(kv_seen)) / float(
                        w.kv_heads * lens.clip(0, w.Skv).sum())
                row["GB/s"] = nbytes / (ms * 1e-3) / 1e9
            rows.append(row)
        del tms, tbs, fns
        torch.cuda.empty_cache()
    return rows


def strip_comments(text: str) -> str:
    """C/C++ source without its comments and empty lines, each line's runs of
    blanks outside literals cut to one space and its ends trimmed (string and
    character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in " \t":
            if not out or out[-1] != " ":
                out.append(" ")
            i += 1
        else:
            out.append(c)
            i += 1
    lines = (l.strip() for l in "".join(out).split("\n"))
    return "\n".join(l for l in lines if l)


def kernel_code_sha256(files) -> str:
    """SHA-256 over the named csrc files with comments removed: a profile's
    counters stay attached to the code they measured through comment edits,
    and detach on any change to the code itself."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        src = os.path.join(ROOT, "transformer_scaled_dot_attn_amd", "csrc", f)
        h.update(strip_comments(open(src, encoding="utf-8").read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 summary of this kernel
    and workload (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known
    size), or None when there is none or the kernel's code has changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in (
                "traffic_bytes_per_launch", "kernel_sources", "kernel_code_sha256"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    if len(fields) != 3:
        return None
    files = fields["kernel_sources"].split()
    csrc = os.path.join(ROOT, "transformer_scaled_dot_attn_amd", "csrc")
    if not all(os.path.exists(os.path.join(csrc, f)) for f in files):
        return None
    if kernel_code_sha256(files) != fields["kernel_code_sha256"]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 20 warm-up steps (~17 ms): the first ~15 steps after a cold start run
    # through a power-management transient (prefill 150 -> 190 -> 150 us)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--parts", default="prefill,decode,masks,gqa,configs,sweep",
                    help="comma list of prefill, decode, masks, copy, gqa, gqa8, configs, sweep "
                         "(default prefill,decode,masks,gqa,configs,sweep); configs times the other "
                         "bf16 prefill workloads; masks times the step's workloads again with "
                         "allowed-masks; gqa8 is the 8-K/V-head decode alone; copy adds a plain 1 GiB device-to-device copy per "
                         "step, the known-size kernel that scales the HBM byte counters; gqa "
                         "measures decode at 32, 8 and 1 K/V heads for 32 query heads; sweep "
                         "measures causal prefill over S = 128 .. 8192 (both reported beside "
                         "the step, under their own keys)")
    ap.add_argument("--headline-first", action="store_true",
                    help="time the step before the other parts (default: after them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads for the CPU baseline (default: every CPU the "
                         "process may use)")
    return ap.parse_args()


def host_cores():
    """(logical CPUs of the host, CPUs this process may run on)."""
    n = os.cpu_count() or 1
    try:
        return n, len(os.sched_getaffinity(0))
    except AttributeError:
        return n, n


def cpu_baseline(threads: int):
    """The float64 CPU oracle (as it stands, one thread per (b, h) slice up
    to `threads`) timed on every configuration: the tiny fp32 causal problem,
    mha768 and prefill4096 whole, padded2048 on 4 heads of each batch item,
    decode8192 on 2 heads of each batch item (a bounded sample: about 10 s of
    CPU work in all).  Prefill rows give GFLOP/s of 4*d flops per visible
    pair, the decode row GB/s of the bytes the decode reads and writes (valid
    K/V rows, q, out, lengths).  Returns the prefill4096 row (the headline's
    workload) with every row under "configs"."""
    import oracle
    import workloads as W
    nproc, usable = host_cores()

    def run(name, pairs=None):
        w = W.WORKLOADS[name]
        x = W.make_inputs(w, pairs)
        lens = x["kv_lens"]
        t0 = time.perf_counter()
        oracle.attention(x["q"], x["k"], x["v"], x["scale"], w.causal, lens, nthreads=threads)
        dt = time.perf_counter() - t0
        slices = x["q"].shape[0] * x["q"].shape[1]
        sub = W.Workload(name, x["q"].shape[0], x["q"].shape[1], w.Sq, w.Skv, w.d, w.dtype,
                         w.causal, w.seed, Hkv=x["k"].shape[1])
        row = {"workload": name, "seconds": dt, "threads": min(threads, slices),
               "sample": "all (b, h) slices" if pairs is None else
               f"{len(pairs)} of {w.B * w.H} (b, h) slices"}
        if w.Sq == 1:
            row["GB/s"] = decode_bytes(sub, lens) / dt / 1e9
        else:
            row["GFLOP/s"] = prefill_flops(sub, lens) / dt / 1e9
        return row

    rows = [run("tiny_f32"), run("mha768_bf16"), run(PREFILL),
            run("padded2048_bf16", [(b, h) for b in range(8) for h in (0, 8, 16, 24)]),
            run(DECODE, [(b, h) for b in range(64) for h in (0, 16)])]
    head = rows[2]
    return {"value": head["GFLOP/s"] / 1e3, "unit": "TFLOP/s", "cores": head["threads"],
            "nproc": nproc, "usable_cpus": usable, "kind": "oracle",
            "sample": f"all 32 heads of {PREFILL} (B=1, S=4096, d=128, causal), float64, "
                      f"{head['seconds']:.2f} s wall on {head['threads']} threads",
            "configs": rows}


def sweep_slopes(rows):
    """Exponent of time in S from the prefill sweep: log2 of the time ratio
    of each doubling, and the least-squares slope of log time on log S over
    S >= 1024 (exercise D of "Attention from First Principles", section 10:
    the work grows as S^2)."""
    pts = [(r["S"], r["ms_per_call"]) for r in rows]
    seg = [{"from": a[0], "to": b[0], "exponent": math.log2(b[1] / a[1])}
           for a, b in zip(pts, pts[1:])]
    big = [(math.log2(S), math.log2(t)) for S, t in pts if S >= 1024]
    fit = None
    if len(big) >= 2:
        mx = sum(x for x, _ in big) / len(big)
        my = sum(y for _, y in big) / len(big)
        fit = sum((x - mx) * (y - my) for x, y in big) / sum((x - mx) ** 2 for x, _ in big)
    return {"per_doubling": seg, "fit_S_ge_1024": fit}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the attention kernels run on a single MI355X "
              "and there is no multi-GPU path (pass --gpus 1).", file=sys.stderr)
        sys.exit(2)
    parts = [p.strip() for p in args.parts.split(",") if p.strip()]

    import numpy as np
    import torch
    import transformer_scaled_dot_attn_amd as attn
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    runs = []
    if "prefill" in parts:
        w = W.WORKLOADS[PREFILL]
        print(f"[bench] preparing {w.name}", file=sys.stderr, flush=True)
        x = W.device_inputs(w, dev, digest=True)
        out = torch.empty_like(x["q"])
        runs.append(("prefill", w, x, out))
    if "decode" in parts:
        w = W.WORKLOADS[DECODE]
        print(f"[bench] preparing {w.name}", file=sys.stderr, flush=True)
        x = W.device_inputs(w, dev, digest=True)
        out = torch.empty_like(x["q"])
        runs.append(("decode", w, x, out))

    copy_src = copy_dst = None
    if "copy" in parts:
        copy_src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    def step():
        for _, w, x, out in runs:
            attn.fwd(x["q"], x["k"], x["v"], out, causal=w.causal, kv_lens=x["kv_lens"],
                     scale=x["scale"])
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    extra = {}

    def secondary(key, what, fn):
        # a failing secondary measurement is reported under its key; the step
        # and its JSON line still follow
        print(f"[bench] {what}", file=sys.stderr, flush=True)
        try:
            extra[key] = fn()
        except Exception as e:  # noqa: BLE001 -- reported, not hidden
            print(f"[bench] {what} failed: {e!r}", file=sys.stderr, flush=True)
            extra[key] = {"error": repr(e)}

    def secondary_parts():
        if "gqa" in parts:
            have = {w.name: x for kind, w, x, _ in runs if kind == "decode"}
            secondary("gqa_decode", "grouped-head decode sweep",
                      lambda: gqa_decode_sweep(attn, W, dev, args.steps, args.warmup, have=have))
        elif "gqa8" in parts:
            secondary("gqa_decode", "8-K/V-head decode",
                      lambda: gqa_decode_sweep(attn, W, dev, args.steps, args.warmup,
                                               names=("gqa_decode8192_bf16",)))
        if "masks" in parts and runs:
            secondary("masks", "allowed-mask runs",
                      lambda: mask_runs(attn, W, runs, args.steps, args.warmup))
        if "configs" in parts:
            secondary("prefill_configs", "other prefill workloads",
                      lambda: prefill_configs(attn, W, dev, args.steps, args.warmup))
        if "sweep" in parts:
            secondary("prefill_sweep", "prefill S sweep",
                      lambda: prefill_sweep(attn, W, dev, args.steps, args.warmup))
            if isinstance(extra.get("prefill_sweep"), list):
                extra["prefill_sweep_slope"] = sweep_slopes(extra["prefill_sweep"])

    # The secondary measurements run first by default, so the step's timed
    # region starts on a GPU already under load (see --headline-first).
    if not args.headline_first:
        secondary_parts()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    attn.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = kernel_stats(attn, ("prefill_bf16_mfma", "decode_bf16_partial", "decode_bf16_combine"))
    step_prefill_us = [round(1e3 * t, 1) for t in attn.profile_samples("prefill_bf16_mfma")]
    attn.profile_enable(False)
    ms_per_step = wall * 1e3 / args.steps

    def avg_ms(name):
        return st[name]["ms"]

    result = {
        "metric": "attn fwd TFLOP/s (causal prefill) + KV-read GB/s (decode), 1×MI355X",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": " + ".join(w.name for _, w, _, _ in runs)},
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    for kind, w, x, out in runs:
        cfg = {"B": w.B, "H": w.H, "Sq": w.Sq, "Skv": w.Skv, "d": w.d, "causal": w.causal}
        if kind == "prefill":
            flops = prefill_flops(w, x["kv_lens_host"])
            kms = avg_ms("prefill_bf16_mfma")
            tflops = flops / (kms * 1e-3) / 1e12
            result["value"] = tflops
            result["config"]["prefill"] = cfg
            cfg["sha256"] = x["sha256"]
            result["roofline"] = {
                "kernel": "prefill_bf16_mfma", "bound": "mfma", "achieved": tflops,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                "traffic": profiled_traffic("prefill_bf16_mfma", w.name),
                "algorithmic_flop_per_launch": flops, "avg_launch_ms": kms,
                "median_us": st["prefill_bf16_mfma"]["median_us"],
                "min_us": st["prefill_bf16_mfma"]["min_us"],
                "launch_us": step_prefill_us}
        else:
            lens = x["kv_lens_host"]
            nbytes = decode_bytes(w, lens)
            p_ms = avg_ms("decode_bf16_partial")
            c_ms = avg_ms("decode_bf16_combine")
            c_ms = 0.0 if math.isnan(c_ms) else c_ms
            kv_bytes = nbytes - 2 * 2 * w.B * w.H * w.d  # what the partial kernel reads
            gbs_op = nbytes / ((p_ms + c_ms) * 1e-3) / 1e9
            gbs_k = kv_bytes / (p_ms * 1e-3) / 1e9
            cfg["kv_len_range"] = list(w.kv_len_range)
            cfg["sum_kv_len"] = int(np.sum(lens))
            cfg["sha256"] = x["sha256"]
            result["config"]["decode"] = cfg
            result["decode"] = {
                "metric": "KV-read GB/s (decode)", "value": gbs_op, "unit": "GB/s",
                "ms_per_call": p_ms + c_ms,
                "roofline": {
                    "kernel": "decode_bf16_partial", "bound": "hbm", "achieved": gbs_k,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs_k / PEAK_HBM_GBS,
                    "traffic": profiled_traffic("decode_bf16_partial", w.name),
                    "algorithmic_bytes_per_launch": kv_bytes,
                    "avg_launch_ms": p_ms,
                    "median_us": st["decode_bf16_partial"]["median_us"],
                    "min_us": st["decode_bf16_partial"]["min_us"]},
                "combine_avg_launch_ms": c_ms,
                "median_us": st["decode_bf16_partial"]["median_us"] +
                (st["decode_bf16_combine"]["median_us"] or 0.0),
                "min_us": st["decode_bf16_partial"]["min_us"] +
                (st["decode_bf16_combine"]["min_us"] or 0.0),
                "combine_launches": st["decode_bf16_combine"]["n"],
            }
    if result["value"] is None and "decode" in result:
        result["value"] = result["decode"]["value"]
        result["unit"] = "GB/s"
        result["roofline"] = result["decode"]["roofline"]

    if args.headline_first:
        secondary_parts()
    result.update(extra)

    if not args.no_cpu_baseline and "prefill" in parts:
        threads = args.cpu_threads or host_cores()[1]
        print(f"[bench] cpu baseline with {threads} threads", file=sys.stderr, flush=True)
        try:
            result["cpu_baseline"] = cpu_baseline(threads)
        except Exception as e:  # noqa: BLE001 -- reported in the line, which still prints
            print(f"[bench] cpu baseline failed: {e!r}", file=sys.stderr, flush=True)
            result["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
