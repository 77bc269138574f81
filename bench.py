"""Benchmark: decode steps over a 2-bit PatternKV-packed KV cache on one MI355X.

Workload (the Llama-3-8B-shaped 32k-context decode configuration): batch 8,
32 q-heads / 8 kv-heads (GQA 4), head_dim 128, bf16 K/V/q, 2-bit codes in
groups of 32 channels, 32 k-means patterns per head, V threshold alpha 0.05,
Chebyshev window 128, context 32768.  One step is one decode step of a
32-layer stack: for every layer, encode-append the new token's K and V
(update_patterns on) and run single-query decode attention over the packed
cache.  The 32 layer caches (6.9 GB) are distinct buffers, so the 256 MB
Infinity Cache cannot hold them.

value = algorithmic bytes of a step / step time (effective GB/s); the bytes
are the packed cache records and pattern tables read by attention, the new
K/V read and records written by encode, q and the outputs.  The roofline
object covers the step's dominant kernel (the one-launch decode step, the only
kernel of the timed region), timed with one event pair on the stream it runs
on around the whole timed region.  A bulk (prefill-style) encode rate is
reported as encode tokens/s.  The CPU oracle is timed on a bounded sample, on
one core and on every usable core.

Usage: python bench.py [--steps K] [--warmup W] [--context T] [--layers L]
       [--no-cpu-baseline] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn effective GB/s over 2-bit packed KV (% of HBM peak); encode tok/s"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attention.json")


# Other workload shapes, measured as attention calls (HIP events over 10 calls
# after 3 warm-up calls); the caches are filled by the bulk encode.
ATTN_CONFIGS = {
    "long4bit": dict(B=1, Hq=32, H=8, T=131072, bits=4, group=64, P=64, mode="pattern"),
    "kvarn": dict(B=64, Hq=32, H=8, T=16384, bits=2, group=32, P=0, mode="kvarn"),
    # the same breadth workload in the NSN scalar mode (52-byte records)
    "nsn": dict(B=64, Hq=32, H=8, T=16384, bits=2, group=32, P=0, mode="nsn"),
    "qwen": dict(B=32, Hq=28, H=4, T=32768, bits=2, group=32, P=64, mode="pattern"),
    # K per channel over 128-token blocks (PatternKV's KIVI-style setting): the
    # 32k context plus 64 tokens in the open block
    "kivi": dict(B=8, Hq=32, H=8, T=32832, bits=2, group=32, P=32, mode="pattern", kch=True),
}


def calib_kernels(mib, dev):
    """Plain kernels of known HBM traffic on `mib` MiB (4 reads: sum; 4 writes:
    fill; 4 copies: negation), whose counters calibrate an attention run's."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        src.sum()
    for _ in range(4):
        dst.fill_(2.0)
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"calib-copy: {mib} MiB x 4 reads, 4 writes, 4 copies")


def attn_config_bytes(c):
    """Algorithmic bytes of one attention call on an ATTN_CONFIGS shape."""
    D, B, Hq, H, T = 128, c["B"], c["Hq"], c["H"], c["T"]
    idx = 2 if c["mode"] == "kvarn" else 4 if c["mode"] == "nsn" else 1
    rec = D * c["bits"] // 8 + (D // c["group"]) * 4 + idx
    if c.get("kch"):
        # K: codes + index per token, one (s, z) word per channel and complete
        # block, binary16 residuals of the open block; V per token as usual
        closed = T // 128 * 128
        k_bytes = T * (D * c["bits"] // 8 + 1) + closed // 128 * D * 4 + (T - closed) * D * 2
        return B * H * (k_bytes + T * rec) + 2 * B * H * c["P"] * D * 4 + B * Hq * D * 6
    return 2 * B * H * T * rec + 2 * B * H * c["P"] * D * 4 + B * Hq * D * 6


def attn_config(name, calib_mib=0):
    import torch

    from bit_kv_cache_encode_amd import KVCache, synth
    c = ATTN_CONFIGS[name]
    dev = torch.device("cuda", 0)
    D = 128
    B, Hq, H, T = c["B"], c["Hq"], c["H"], c["T"]
    k, v = synth.device_kv(B, H, T, D, device=dev)
    kch = c.get("kch", False)
    cache = KVCache(B, Hq, H, T + 64, bits=c["bits"], group=c["group"], mode=c["mode"],
                    max_patterns=max(c["P"], 1), device=dev, k_per_channel=kch)
    if c["mode"] == "pattern":
        cache.init_patterns(k[:, :, :2048].contiguous(), v[:, :, :2048].contiguous(), c["P"])
    else:
        cache.init_patterns(k[:, :, :1024].contiguous(), v[:, :, :1024].contiguous(), 0)
    cache.encode_append(k, v)
    del k, v
    q = synth.device_queries(B, Hq, D, device=dev)
    out = torch.empty((B, Hq, D), device=dev)
    for _ in range(10):
        cache.attn_decode(q, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 50
    e0.record()
    for _ in range(n):
        cache.attn_decode(q, out=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    if not kch:
        assert cache.layout.record_bytes == (D * c["bits"] // 8 + (D // c["group"]) * 4
                                             + (2 if c["mode"] == "kvarn" else
                                                4 if c["mode"] == "nsn" else 1))
    nbytes = attn_config_bytes(c)
    res = {"attn_config": name, "shape": c, "us_per_call": round(us, 2),
           "algorithmic_bytes": nbytes, "effective_GBs": round(nbytes / us / 1e3, 1),
           "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    if kch:
        # a decode step here is the append of one token (encode, the open
        # block's residual write) and the attention: separate launches
        kn, vn = synth.device_kv(B, H, 1, D, layer=1, device=dev)
        steps = 10
        e0.record()
        for _ in range(steps):
            cache.decode_step(kn, vn, q, out=out)
        e1.record()
        torch.cuda.synchronize()
        res["decode_step_us"] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    print(json.dumps(res))
    if calib_mib:
        calib_kernels(calib_mib, dev)


def streaming(args):
    """The streaming-accumulation workload: a Qwen2.5-7B-shaped layer (28 q / 4
    kv heads, head_dim 128), batch 32, a 32768-token prefix, then 256 decode
    steps (append one token with the Chebyshev window on, then attend) whose K
    mean drifts (step j adds 0.01 j u, u ~ N(0, I) per unit); 2-bit group 32,
    64 k-means patterns growing by one per 128 decode steps.  Prints one JSON
    line: the time per step, and at sampled steps the error of the quantised
    attention against fp32 attention over the unquantised inputs (max abs and
    relative L2 over every (batch, q-head) output), GPU-vs-oracle parity on
    one unit, and V utilisation (the share of V vectors that keep their
    pattern under the section 3.3 threshold)."""
    import numpy as np
    import torch

    import oracle as O
    from bit_kv_cache_encode_amd import KVCache, synth

    dev = torch.device("cuda", 0)
    B, Hq, H, D, T0, S, P, W = 32, 28, 4, 128, args.context, 256, 64, 128
    gq = Hq // H
    k, v = synth.device_kv(B, H, T0 + S, D, device=dev, dtype=torch.float32)
    drift = torch.from_numpy(synth.drift_dirs(B, H, D)).to(dev)
    ramp = torch.arange(1, S + 1, device=dev, dtype=torch.float32)
    k[:, :, T0:] += 0.01 * ramp[None, None, :, None] * drift[:, :, None, :]
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    cache = KVCache(B, Hq, H, T0 + S, bits=2, group=32, mode="pattern", max_patterns=P + 2,
                    pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16, device=dev)
    cache.init_patterns(k[:, :, :2048].contiguous(), v[:, :, :2048].contiguous(), P)
    cache.encode_append(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
    qs = [synth.device_queries(B, Hq, D, step=s, device=dev) for s in range(S)]
    kn = [k[:, :, T0 + s:T0 + s + 1].contiguous() for s in range(S)]
    vn = [v[:, :, T0 + s:T0 + s + 1].contiguous() for s in range(S)]
    sample = sorted({0, 63, 127, 128, 191, S - 1})
    out = torch.empty((B, Hq, D), device=dev)
    saved = {}
    # timed pass: the 256 steps back to back, outputs of sampled steps kept
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(S):
        cache.decode_step(kn[s], vn[s], qs[s], out=out)
        if s in sample:
            saved[s] = out.clone()
    e1.record()
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / S
    vidx = cache.region("v_idx").view(B * H, -1)[:, :T0 + S].cpu().numpy()
    # exact fp32 attention over the unquantised (bf16) inputs, per sampled step
    kf = k.float().view(B * H, T0 + S, D)
    vf = v.float().view(B * H, T0 + S, D)
    records = []
    # one unit through the oracle
    ref = O.RefCache(1, gq, 1, D, T0 + S, bits=2, group=32, mode=O.PATTERN, max_patterns=P + 2,
                     pattern_window=W, v_alpha=0.05, in_dtype=O.IN_BF16)
    ku = k[0:1, 0:1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    vu = v[0:1, 0:1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ref.init_patterns(ku[:, :, :2048], vu[:, :, :2048], P)
    ref.encode_append(ku[:, :, :T0], vu[:, :, :T0])
    for s in range(S):
        ref.encode_append(ku[:, :, T0 + s:T0 + s + 1], vu[:, :, T0 + s:T0 + s + 1], update=1)
        if s not in sample:
            continue
        n = T0 + s + 1
        q = qs[s].float().view(B * H, gq, D)
        kt = kf[:, :n].transpose(1, 2).contiguous()
        sc = torch.matmul(q, kt) / (D ** 0.5)
        pr = torch.softmax(sc, dim=-1)
        exact = torch.matmul(pr, vf[:, :n].contiguous()).view(B, Hq, D)
        del kt, sc, pr
        got = saved[s]
        diff = (got - exact).abs()
        want_u = ref.attn_decode(qs[s][0:1, 0:gq].contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        par = float(np.abs(got[0:1, 0:gq].cpu().numpy() - want_u).max())
        used = vidx[:, :n]
        dec = vidx[:, T0:n]
        records.append({
            "step": s, "tokens": n, "patterns": None,
            "max_abs_err_vs_fp32": round(float(diff.max()), 5),
            "rel_l2_err_vs_fp32": round(float(diff.norm() / exact.norm()), 5),
            "gpu_vs_oracle_unit0": float(f"{par:.3e}"),
            "v_utilisation_all": round(float((used != 0xFF).mean()), 4),
            "v_utilisation_decode": round(float((dec != 0xFF).mean()), 4)})
    for r in records:
        r["patterns"] = P + (r["step"] + 1) // W
    assert cache.n_patterns == P + S // W and ref.n_patterns == cache.n_patterns
    res = {"mode": "streaming",
           "workload": (f"Qwen2.5-7B-shaped layer: batch {B}, {Hq} q / {H} kv heads, head_dim {D}, "
                        f"prefix {T0}, then {S} decode steps (append 1 token with the Chebyshev "
                        f"window {W} on + attention) with drifting K mean; 2-bit group 32, "
                        f"{P} k-means patterns -> {cache.n_patterns}"),
           "us_per_step": round(us_step, 2), "steps": S,
           "errors": "max abs and relative L2 over all (batch, q-head) outputs against fp32 "
                     "attention over the unquantised bf16 inputs; gpu_vs_oracle on unit (0, 0)",
           "records": records}
    print(json.dumps(res))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--kmeans-tokens", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-patterns", action="store_true",
                    help="one pattern table and Chebyshev window per kv-head for the whole batch")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--split-step", action="store_true",
                    help="run each layer's step as two calls (encode-append, then attention) "
                         "instead of the one-launch kvq_decode_step")
    ap.add_argument("--attn-only", type=int, default=0,
                    help="profiling aid: run N launches of the step's dominant kernel (the "
                         "one-launch step, or with --split-step the attention) and exit")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="with --attn-only: then run plain kernels of known traffic on this many "
                         "MiB (4 reads: sum; 4 writes: fill; 4 copies: negation), whose HBM "
                         "counters calibrate the attention's")
    ap.add_argument("--attn-config", choices=sorted(ATTN_CONFIGS),
                    help="secondary measurement: decode attention alone on another workload "
                         "shape (long4bit: B 1, 131072 tokens, 4-bit G64, 64 patterns; "
                         "kvarn: 64 samples x 16384, KVarN 2-bit; qwen: B 32, 28 q / 4 kv "
                         "heads, 32768 tokens, 64 patterns; nsn: the kvarn shape in the NSN "
                         "scalar mode; kivi: the step's shapes with K "
                         "quantised per channel over 128-token blocks, 32832 tokens); prints one "
                         "JSON line")
    ap.add_argument("--streaming", action="store_true",
                    help="the streaming-accumulation workload (Qwen2.5-7B shape, batch 32, "
                         "32768-token prefix, 256 drifting decode steps): per-step time and, at "
                         "sampled steps, error against fp32 attention, oracle parity on one unit "
                         "and V utilisation; prints one JSON line")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "RAW_DIR"),
                    help="no GPU: summarise three rocprofv3 --pmc runs of --attn-only N "
                         "--calib-copy M (FETCH_SIZE; WRITE_SIZE; TCC_EA0_RDREQ 32B/64B/128B) "
                         "into profiles/traffic_attention.json")
    return ap.parse_args()


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn.hip", "attn_mfma.hip", "attn_mfma_common.h", "encode_vec.h", "kvq_internal.h"):
        p = os.path.join(ROOT, "bit_kv_cache_encode_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_summary(args):
    """Attention HBM bytes per launch from rocprofv3 counter CSVs, calibrated
    against kernels of known traffic run in the same process."""
    import csv
    import glob

    def rows(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert f, f"no counter_collection.csv under {d}"
        return list(csv.DictReader(open(f[0])))

    def per_dispatch(rs, counter, pred):
        vals = {}
        for r in rs:
            if r["Counter_Name"] == counter and pred(r["Kernel_Name"]):
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return list(vals.values())

    attn = lambda n: "attn_mfma_kernel" in n or "attn_split_kernel" in n
    red = lambda n: "reduce_kernel" in n
    fill = lambda n: "FillFunctor" in n
    fr, wr, rr = rows(args.traffic_from[0]), rows(args.traffic_from[1]), rows(args.traffic_from[2])
    f_attn = per_dispatch(fr, "FETCH_SIZE", attn)
    w_attn = per_dispatch(wr, "WRITE_SIZE", attn)
    f_red = per_dispatch(fr, "FETCH_SIZE", red)
    w_fill = per_dispatch(wr, "WRITE_SIZE", fill)
    n_calib = args.calib_copy * (1 << 20) if args.calib_copy else None
    assert n_calib, "--traffic-from needs --calib-copy M (the MiB used in the runs)"
    big = lambda xs: [x for x in xs if x * 1024 > 0.25 * n_calib]
    f_red, w_fill = big(f_red), big(w_fill)
    k_read = n_calib / (1024 * sum(f_red) / len(f_red))
    k_write = n_calib / (1024 * sum(w_fill) / len(w_fill))
    fetch_kib = sum(f_attn) / len(f_attn)
    write_kib = sum(w_attn) / len(w_attn)
    raw = {}
    for c in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum",
              "TCC_EA0_RDREQ_sum"):
        v = per_dispatch(rr, c, attn)
        raw[c] = sum(v) / len(v) if v else None
    raw_bytes = None
    if all(raw[c] is not None for c in ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                                        "TCC_EA0_RDREQ_128B_sum")):
        raw_bytes = (32 * raw["TCC_EA0_RDREQ_32B_sum"] + 64 * raw["TCC_EA0_RDREQ_64B_sum"] +
                     128 * raw["TCC_EA0_RDREQ_128B_sum"])
    out = {
        "source_hash": attn_source_hash(),
        "bytes_per_launch": round(fetch_kib * 1024 * k_read + write_kib * 1024 * k_write),
        "fetch_size_kib": round(fetch_kib, 1), "write_size_kib": round(write_kib, 1),
        "read_factor": round(k_read, 4), "write_factor": round(k_write, 4),
        "calibration": f"{args.calib_copy} MiB torch sum (reads) and fill_ (writes)",
        "commands": [
            "cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -o run --output-format csv -- "
            f"python3 -u <repo>/bench.py --attn-only 16 --calib-copy {args.calib_copy}",
            f"rocprofv3 --pmc WRITE_SIZE -d <write_dir> -o run --output-format csv -- "
            f"python3 -u <repo>/bench.py --attn-only 16 --calib-copy {args.calib_copy}",
            f"rocprofv3 --pmc TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum "
            f"TCC_EA0_RDREQ_sum -d <raw_dir> -o run --output-format csv -- "
            f"python3 -u <repo>/bench.py --attn-only 16 --calib-copy {args.calib_copy}",
            f"python bench.py --traffic-from <fetch_dir> <write_dir> <raw_dir> "
            f"--calib-copy {args.calib_copy}"],
        # --attn-only runs on the freshly encoded prefix: T = context tokens,
        # 64 units, 49-byte records, 32 patterns, 8 x 32 query heads
        "algorithmic_bytes_per_launch": 2 * 64 * args.context * 49 + 2 * 64 * 32 * 128 * 4
                                        + 8 * 32 * 128 * 6,
        "dispatches": len(f_attn),
        "raw_read_requests": raw, "raw_read_bytes_per_launch": raw_bytes,
    }
    if args.attn_config:
        # a secondary workload: its attention calls (10 warm-up + 50 timed)
        name = args.attn_config
        out["kernel"] = f"attention (split + combine), {name} workload"
        out["workload"] = ATTN_CONFIGS[name]
        out["algorithmic_bytes_per_launch"] = attn_config_bytes(ATTN_CONFIGS[name])
        out["ratio_to_algorithmic"] = round(out["bytes_per_launch"] / out["algorithmic_bytes_per_launch"], 4)
        out["commands"] = [c.replace("--attn-only 16", f"--attn-config {name}")
                           .replace("--traffic-from", f"--attn-config {name} --traffic-from")
                           for c in out["commands"]]
        dst = os.path.join(ROOT, "profiles", f"traffic_attn_{name}.json")
        json.dump(out, open(dst, "w"), indent=1)
        print(json.dumps(out))
        return
    if not args.split_step:
        # one-launch step over context + 1 tokens: attention bytes plus the
        # new token's encode (K/V in, records out, the two pattern tables)
        out["kernel"] = "decode step in one launch: encode 1 token + attention (split + combine)"
        out["algorithmic_bytes_per_launch"] = (2 * 64 * (args.context + 1) * 49 + 2 * 64 * 32 * 128 * 4
                                               + 8 * 32 * 128 * 6
                                               + 2 * 64 * 128 * 2 + 2 * 64 * 49)
    else:
        out["kernel"] = "attention (split + combine)"
    flag = "" if not args.split_step else " --split-step"
    out["commands"] = [c.replace("--calib-copy", flag.strip() + " --calib-copy").replace("  ", " ")
                       if flag else c for c in out["commands"]]
    dst = os.path.join(ROOT, "profiles", "traffic_attention.json")
    json.dump(out, open(dst, "w"), indent=1)
    print(json.dumps(out))


def main():
    args = parse()
    if args.traffic_from:
        traffic_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by (batch, kv-head) units with no communication, so "
              "one GPU's throughput is measured at its real per-GPU shape)", file=sys.stderr)
        sys.exit(2)
    if args.attn_config:
        attn_config(args.attn_config, args.calib_copy)
        return
    if args.streaming:
        streaming(args)
        return
    import torch

    from bit_kv_cache_encode_amd import KVCache, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B, Hq, H, D, T0, L = args.batch, 32, 8, 128, args.context, args.layers
    P, W = 32, 128
    n_steps = args.warmup + args.steps
    max_tokens = T0 + n_steps + 64
    U = B * H

    # ---- setup (untimed): one layer mined + bulk-encoded, then replicated
    k, v = synth.device_kv(B, H, T0, D, layer=0, device=dev)
    SH = args.shared_patterns
    PU = H if SH else U          # pattern-table units
    base = KVCache(B, Hq, H, max_tokens, bits=2, group=32, mode="pattern", max_patterns=P,
                   pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16, device=dev,
                   shared_patterns=SH)
    nk = min(args.kmeans_tokens, T0)
    kpre, vpre = k[:, :, :nk].contiguous(), v[:, :, :nk].contiguous()
    torch.cuda.synchronize()
    # pattern mining (k-means over the prefix, K and V of every unit), one layer
    i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    i0.record()
    base.init_patterns(kpre, vpre, P)
    i1.record()
    torch.cuda.synchronize()
    init_ms = i0.elapsed_time(i1)
    del kpre, vpre
    # bulk encode rate: the whole prefix in one append (prefill-style)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    base.encode_append(k, v)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1)
    # repeat the bulk encode on a scratch cache to get a warm measurement
    scratch = KVCache(B, Hq, H, T0, bits=2, group=32, mode="pattern", max_patterns=P,
                      pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16, device=dev,
                      shared_patterns=SH)
    tab_shape = (H, P, D) if SH else (B, H, P, D)
    scratch.set_patterns(base.region("k_tab").view(torch.float32).view(tab_shape).clone(),
                         base.region("v_tab").view(torch.float32).view(tab_shape).clone())
    e0.record()
    scratch.encode_append(k, v)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = min(bulk_ms, e0.elapsed_time(e1))
    del scratch, k, v
    layers = [base] + [base.clone() for _ in range(L - 1)]
    torch.cuda.synchronize()

    # per-step inputs: new K/V token per layer, one query per layer
    kn, vn = synth.device_kv(B, H, n_steps * L, D, layer=1, device=dev)
    kn = kn.view(B, H, n_steps, L, D).permute(2, 3, 0, 1, 4).contiguous()
    vn = vn.view(B, H, n_steps, L, D).permute(2, 3, 0, 1, 4).contiguous()
    qs = [synth.device_queries(B, Hq, D, step=s, device=dev) for s in range(L)]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)

    if args.attn_only:
        # the step's dominant kernel: the one-launch step (default) or the
        # attention launch of the two-call form
        for i in range(args.attn_only):
            c = layers[i % L]
            if args.split_step:
                c.attn_decode(qs[i % L], out=out)
            else:
                s_ = i // L
                c.decode_step(kn[s_, i % L][:, :, None, :], vn[s_, i % L][:, :, None, :], qs[i % L],
                              out=out)
        torch.cuda.synchronize()
        print(f"attn-only: {args.attn_only} calls done")
        if args.calib_copy:
            calib_kernels(args.calib_copy, dev)
        return

    rec = base.layout.record_bytes
    in_b = 2

    def attn_bytes(T):
        return 2 * U * T * rec + 2 * PU * P * D * 4 + B * Hq * D * (in_b + 4)

    # the new token's K/V in and its records out; the pattern tables the encode
    # reads are the ones the attention reads in the same launch, counted there
    enc_bytes = 2 * U * D * in_b + 2 * U * rec

    # The one-launch step is the only kernel of the timed region: one event pair
    # on its stream around the whole region gives its average launch duration
    # (with the few-microsecond gaps between back-to-back launches), and so it
    # can never exceed the step time per layer.  The two-call form (a
    # profiling aid) brackets a rotating sample of layers instead (an event
    # record between two launches costs device time of its own): per sampled
    # layer [0] before the encode, [2] between it and the attention, [1] after.
    EV_EVERY = max(1, min(16, L))

    def sampled(s, li):
        return args.split_step and (li - s) % EV_EVERY == 0

    def step(s, ev=None):
        for li, c in enumerate(layers):
            e = ev[li] if ev is not None and sampled(s, li) else None
            if e is not None:
                e[0].record()
            if args.split_step:
                c.encode_append(kn[s, li][:, :, None, :], vn[s, li][:, :, None, :],
                                update_patterns=True)
                if e is not None:
                    e[2].record()
                c.attn_decode(qs[li], out=out)
            else:
                c.decode_step(kn[s, li][:, :, None, :], vn[s, li][:, :, None, :], qs[li], out=out)
            if e is not None:
                e[1].record()

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    T_start = layers[0].n_tokens
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for _ in range(L)] for _ in range(args.steps)]
    stream = torch.cuda.current_stream(dev)    # the stream the library launches on
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for s in range(args.steps):
        step(args.warmup + s, evs[s])
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    region_ms = r0.elapsed_time(r1)
    layer_avg_us = 1e3 * region_ms / (args.steps * L)
    T_mid = T_start + args.steps // 2 + 1
    step_bytes = L * (attn_bytes(T_mid) + enc_bytes)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    if args.split_step:
        # dominant kernel: the attention launch; the encode launch on its own
        used = [evs[s][li] for s in range(args.steps) for li in range(L) if sampled(args.warmup + s, li)]
        attn_avg_us = 1e3 * sum(e[2].elapsed_time(e[1]) for e in used) / len(used)
        enc_avg_us = 1e3 * sum(e[0].elapsed_time(e[2]) for e in used) / len(used)
        kern, kern_us, kern_bytes = "attention (split + combine)", attn_avg_us, attn_bytes(T_mid)
        timing = ("HIP events around the attention launch of a rotating sample of layers "
                  f"(every {EV_EVERY}th) inside the timed steps")
    else:
        # dominant kernel: the one-launch step (encode 1 token + attention)
        kern = "decode step in one launch: encode 1 token + attention (split + combine)"
        kern_us, kern_bytes = layer_avg_us, attn_bytes(T_mid) + enc_bytes
        timing = (f"one HIP event pair on the launch stream around the timed region "
                  f"({args.steps * L} launches, nothing else launched): device time / launches")
        # the single-token encode as its own launch, on a copy of one layer,
        # with the device kept busy while the host queues the launches
        enc_copy = layers[0].clone()
        eev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
        try:
            torch.cuda._sleep(50_000_000)
        except Exception:
            pass
        for i in range(L):
            eev[i][0].record()
            enc_copy.encode_append(kn[i % n_steps, 0][:, :, None, :], vn[i % n_steps, 0][:, :, None, :],
                                   update_patterns=True)
            eev[i][1].record()
        torch.cuda.synchronize()
        enc_avg_us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in eev[1:]) / (L - 1)
        del enc_copy
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        # counters taken on this kernel, sources and table layout
        if tr.get("source_hash") == attn_source_hash() and tr.get("kernel") == kern and not SH:
            traffic = tr.get("bytes_per_launch")

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": (f"decode step of a {L}-layer Llama-3-8B-shaped stack: batch {B}, "
                                f"{Hq} q / {H} kv heads, head_dim {D}, context {T0}, bf16 in, "
                                f"2-bit PatternKV codes (group 32, {P} patterns, alpha 0.05, "
                                f"window {W}"
                                + (", tables shared by the batch" if SH else "")
                                + "); per layer encode-append 1 token + decode attention"
                                + (" (two calls)" if args.split_step else " in one launch")),
                   "batch": B, "context": T0, "layers": L, "n_q_heads": Hq, "n_kv_heads": H,
                   "head_dim": D, "bits": 2, "group": 32, "patterns": P,
                   "shared_patterns": SH},
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kern,
                     "avg_launch_us": round(kern_us, 3), "timing": timing,
                     "algorithmic_bytes_per_launch": kern_bytes},
        "layer_step_avg_us": round(ms_step * 1e3 / L, 3),
        "encode": {"bulk_tok_s": round(B * T0 / (bulk_ms * 1e-3), 1),
                   "bulk_tokens": B * T0, "bulk_ms": round(bulk_ms, 3),
                   "decode_step_tok_s": round(B / (enc_avg_us * 1e-6), 1),
                   "decode_step_avg_us": round(enc_avg_us, 3),
                   "token": "one position's K and V for all 8 kv-heads of one layer"},
        "pattern_init": {"ms": round(init_ms, 3), "prefix_tokens": nk, "patterns": P,
                         "what": ("k-means (binary64) for K and V of each of the "
                                  f"{H} kv-heads of one layer over its {B} prefixes pooled"
                                  if SH else
                                  "k-means (binary64) over the prefix for K and V of all "
                                  f"{U} (batch, kv-head) units of one layer")},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, T0, P, W, attn_bytes, enc_bytes, U)
    print(json.dumps(res))


def _host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cores": usable}


def _oracle_unit_steps(args, T0, P, W, attn_bytes, enc_bytes, U, unit, seconds):
    """Decode steps of one oracle cache (one (batch, kv-head) unit with its 4
    q-heads at the workload's context) until `seconds` of stepping are spent.
    Returns (steps, seconds, bytes)."""
    import oracle as O
    from bit_kv_cache_encode_amd import synth

    D, rep, n_max = 128, 4, 4096
    k = synth.k_vectors(1, 1, T0 + n_max, D, seed=synth.seed_for("k") + 17 * unit)
    v = synth.v_vectors(1, 1, T0 + n_max, D, seed=synth.seed_for("v") + 17 * unit)
    kb, vb = synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v)
    del k, v
    q = synth.f32_to_bf16_bits(synth.queries(1, rep, D, step=unit))
    r = O.RefCache(1, rep, 1, D, T0 + n_max, max_patterns=P, pattern_window=W,
                   in_dtype=O.IN_BF16)
    nk = min(args.kmeans_tokens, T0)
    r.init_patterns(kb[:, :, :nk], vb[:, :, :nk], P)
    r.encode_append(kb[:, :, :T0], vb[:, :, :T0])
    steps, secs, nbytes = 0, 0.0, 0.0
    while secs < seconds and steps < n_max:
        t = T0 + steps
        t_start = time.perf_counter()
        r.encode_append(kb[:, :, t:t + 1], vb[:, :, t:t + 1], update=1)
        r.attn_decode(q)
        secs += time.perf_counter() - t_start
        nbytes += (attn_bytes(t + 1) + enc_bytes) / U
        steps += 1
    return steps, secs, nbytes


def cpu_baseline(args, T0, P, W, attn_bytes, enc_bytes, U):
    """The oracle, as it stands, on a bounded sample of the same workload:
    (batch, kv-head) units at the same context, each stepping decode steps
    (encode 1 token with the Chebyshev window on + 4-q-head attention) for a
    time budget.  Run once on one core, then on every usable core with one
    unit per thread (the oracle is C called through ctypes, which releases the
    interpreter lock, and each unit is an independent cache)."""
    from concurrent.futures import ThreadPoolExecutor

    host = _host_cpu()
    st, ss, sb = _oracle_unit_steps(args, T0, P, W, attn_bytes, enc_bytes, U, 0, args.cpu_seconds)
    single = sb / ss / 1e9
    n = max(1, min(16, host["usable_cores"]))
    t_all = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        res = list(ex.map(lambda i: _oracle_unit_steps(args, T0, P, W, attn_bytes, enc_bytes, U,
                                                       1 + i, args.cpu_seconds), range(n)))
    t_all = time.perf_counter() - t_all
    # aggregate rate: every thread's bytes over the longest thread's stepping time
    tot_bytes = sum(r[2] for r in res)
    span = max(r[1] for r in res)
    return {"value": round(tot_bytes / span / 1e9, 5), "unit": "GB/s", "cores": n,
            "kind": "oracle",
            "single_core_value": round(single, 5),
            "host": host,
            "sample": (f"{n} threads, one (batch, kv-head) unit of the {U} each at context {T0}, "
                       f"{sum(r[0] for r in res)} decode steps in all (encode 1 token + 4-q-head "
                       f"attention), {span:.1f} s of stepping per thread ({t_all:.1f} s with set-up); "
                       f"single core: {st} steps in {ss:.1f} s; C oracle, bytes counted as in value")}


if __name__ == "__main__":
    main()
