#!/usr/bin/env python3
"""Benchmark of the OSCAR INT2 KV-cache hot path on one MI355X.

Default workload (the headline configuration): Qwen3-8B-shaped attention,
36 layers, each with its own calibrated R_K, R_V and clips; 32 query / 8 KV
heads, head_dim 128; batch 1 at a 32768-token context (16 sink + 128 recent
BF16 tokens, the rest INT2 with G = 64, fp16 scale / zero); 16-token pages in
a shuffled page table.  One step is one generation step of the attention
stack: for every layer, write-on-append of the new token (the token leaving
the recent window is rotated, clipped and packed into history) followed by
the mixed-precision paged decode.  The step is captured once in a HIP graph
and replayed; sequence lengths advance on the device each replay.

`--workload bs64` runs the batch-64 configuration (per-request lengths
uniform in [8192, 32768], pages of all requests interleaved in one pool).

`--workload extend` runs the extend (chunked-prefill) attention: per layer, a
4096-token chunk attends to its 28672-token cached prefix and causally to
itself (Qwen3-8B-shaped, 36 layers, G = 64); its line names its own metric
(TFLOP/s against the matrix-core peak).

`--workload write` runs the fused write path at prefill (Qwen3-4B-shaped,
36 layers, 32 q / 8 KV heads, G = 32): one step writes 8 prompts x 32768 new
tokens into every layer's cache (rotate, clip, INT2-pack, page-store; sink and
recent kept bf16); then 64 decode steps with write-on-append of each new
token are timed as well.  Its line names its own metric (write GB/s).

`--workload 28x100k` runs the capacity workload (Qwen3-32B-shaped, 64 layers,
28 requests x 100000 tokens, GQA 8, G = 128, ~104 GB of INT2 cache; its
all-BF16 copy does not fit one GPU), `--workload int4_28x100k` the same
tokens from an INT4 cache (~195 GB: the 4-bit comparison point of the
capacity result), and `--workload
config0` the single-layer 4096-token correctness configuration (8 query / 2
KV heads, G = 32).

The default run (no --workload) times bs1 -- its `value` -- and adds every
other workload's line under its name ("bs64", "28x100k", "int4_28x100k",
"write", "extend", "config0"), each with its own roofline and CPU oracle baseline, plus the
measured read ceilings of the device ("read_ceiling": streaming and
page-gather reads by oscar_read_probe), against which each bandwidth-bound
roofline also reports `frac_of_measured_ceiling`.

Printed: one JSON line (metric, value in GB/s of algorithmic bytes per step,
tokens/s, per-replay median / p10 / p90, the in-run BF16 paged-decode
comparison, the roofline of the dominant kernel and the CPU oracle baseline
with the host's core count and CPU model).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "INT2 decode-attn KV GB/s (% HBM peak) + tokens/s, 32K ctx bs1 & bs64"
HBM_PEAK_GBS = 8000.0
HEAD_DIM = 128


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["bs1", "bs64", "write", "28x100k", "int4_28x100k", "extend", "config0"],
                   default=None,
                   help="default: bs1, with every other workload's figures added to its line")
    p.add_argument("--no-companion", action="store_true", help="default run: bs1 alone")
    p.add_argument("--layers", type=int, default=None, help="override the layer count (testing only)")
    p.add_argument("--seed", type=int, default=1)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-bf16", action="store_true")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter scale reference)")
    p.add_argument("--traffic-from", nargs=5, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                       "COPY_WRITE_CSV"),
                   help="only turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files of a run of WORKLOAD and "
                        "of --copy-probe-mb into per-launch HBM bytes of its dominant kernel, stored in "
                        "profiles/hbm_traffic.json")
    return p.parse_args()


# ------------------------------------------------------------ HBM traffic
# Measured HBM bytes per launch of each workload's dominant kernel, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled
# by what the same counter reports for a plain device copy of known size.  An
# entry is used only while the kernel's sources are the ones it was measured
# on (their SHA-256 is stored with it).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# (the device code of each kernel: its source and the headers with device
# code; kernels.h only declares the host-side launchers)
DOMINANT = {"bs1": ("attend_kernel", ["decode_int2.hip", "attn_common.h", "common.h"]),
            "bs64": ("attend_kernel", ["decode_int2.hip", "attn_common.h", "common.h"]),
            "write": ("write_hist_kernel", ["write.hip", "common.h"]),
            "extend": ("extend_kernel", ["extend.hip", "attn_common.h", "common.h"]),
            "28x100k": ("attend_kernel", ["decode_int2.hip", "attn_common.h", "common.h"]),
            "int4_28x100k": ("attend_kernel", ["decode_int2.hip", "attn_common.h", "common.h"]),
            "config0": ("attend_kernel", ["decode_int2.hip", "attn_common.h", "common.h"])}


def kernel_sources_sha(workload):
    import hashlib
    h = hashlib.sha256()
    for f in DOMINANT[workload][1]:
        with open(os.path.join(ROOT, "bit_rotated_kv_oscar_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel, or None when
    not measured on the current sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            e = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not e or e.get("sources_sha256") != kernel_sources_sha(workload):
        return None
    return int(e["hbm_bytes_per_launch"])


def traffic_from(args):
    import csv

    workload, f_csv, w_csv, cf_csv, cw_csv = args.traffic_from
    kname = DOMINANT[workload][0]

    def mean_kib(path, pattern):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if pattern in r["Kernel_Name"]]
        return sum(vals) / len(vals), len(vals)

    copy_bytes = 1024 * (1 << 20)
    fc, _ = mean_kib(cf_csv, "copyBuffer")
    wc, _ = mean_kib(cw_csv, "copyBuffer")
    fetch_scale, write_scale = copy_bytes / (fc * 1024), copy_bytes / (wc * 1024)
    fk, nf = mean_kib(f_csv, kname)
    wk, nw = mean_kib(w_csv, kname)
    fetch_b, write_b = fk * 1024 * fetch_scale, wk * 1024 * write_scale
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    data[workload] = {"kernel": kname, "sources_sha256": kernel_sources_sha(workload),
                      "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
                      "fetch_bytes_per_launch": int(round(fetch_b)), "write_bytes_per_launch": int(round(write_b)),
                      "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                      "dispatches": [nf, nw],
                      "copy_probe": {"bytes": copy_bytes, "fetch_kib": round(fc, 1), "write_kib": round(wc, 1),
                                     "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)}}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(data[workload]))


WORKLOADS = {
    "bs1": dict(name="qwen3-8b-shaped attention decode, 36 layers, batch 1, context 32768, G 64",
                layers=36, hq=32, hkv=8, G=64, batch=1, len_lo=32768, len_hi=32768),
    "bs64": dict(name="qwen3-8b-shaped attention decode, 36 layers, batch 64, contexts U[8192, 32768], G 64",
                 layers=36, hq=32, hkv=8, G=64, batch=64, len_lo=8192, len_hi=32768),
    "write": dict(name="qwen3-4b-shaped fused KV write at prefill, 36 layers, 8 prompts x 32768 tokens, G 32",
                  layers=36, hq=32, hkv=8, G=32, batch=8, len_lo=32768, len_hi=32768),
    # ~104 GB of INT2 cache (64 layers x 1.63 GB) on one GPU; its all-BF16
    # copy (734 GB) does not fit, so this workload has no in-run BF16 ratio
    "28x100k": dict(name="qwen3-32b-shaped attention decode, 64 layers, 28 requests x 100000-token context, G 128",
                    layers=64, hq=64, hkv=8, G=128, batch=28, len_lo=100000, len_hi=100000,
                    bf16_bytes_note="all-BF16 cache of the same tokens: 734 GB, beyond one GPU's 288 GB"),
}
# the same tokens from an INT4 cache (~195 GB): the pages' 4-bit comparison
# point of the capacity result, which fits the 288 GB of one MI355X
WORKLOADS["int4_28x100k"] = dict(
    name="qwen3-32b-shaped attention decode from an INT4 cache, 64 layers, 28 requests x 100000-token context, "
         "G 128", layers=64, hq=64, hkv=8, G=128, batch=28, len_lo=100000, len_hi=100000, bits=4,
    bf16_bytes_note="all-BF16 cache of the same tokens: 734 GB, beyond one GPU's 288 GB")
# the single-layer correctness configuration (cache-resident: a latency
# figure, not a bandwidth result); pages contiguous
WORKLOADS["config0"] = dict(name="single layer, batch 1, 8 q / 2 KV heads, context 4096 (16 sink + 128 recent BF16 + "
                                 "3952 INT2), G 32, one decode step", layers=1, hq=8, hkv=2, G=32, batch=1,
                            len_lo=4096, len_hi=4096, contiguous_pages=True)
WRITE_METRIC = "INT2 fused KV write GB/s (% HBM peak) + tokens/s, prefill 8 x 32K, 36 layers"
WORKLOADS["extend"] = dict(
    name="qwen3-8b-shaped extend attention (chunked prefill) over a cached INT2 + BF16 prefix, 36 layers, "
         "batch 1, prefix 28672 + chunk 4096, G 64",
    layers=36, hq=32, hkv=8, G=64, batch=1, len_lo=28672, len_hi=28672, chunk=4096)
EXTEND_METRIC = "INT2 extend-attn TFLOP/s (% MFMA peak) + tokens/s, prefix 28672 + chunk 4096, 36 layers"
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix-core peak


def n_hist_tokens(L):
    return max(0, L - 144)


def decode_bytes(lens, hq, hkv, G, bits=2):
    """Algorithmic bytes of one decode call: INT2 (or INT4) codes + fp16 meta
    of every history token, raw bf16 sink/recent tokens, page-table entries,
    q, out, and R_K / R_V (fp32) once."""
    per_tok_int2 = 2 * (16 * bits + 4 * (128 // G))
    b = 0
    for L in lens:
        nh = n_hist_tokens(L)
        b += nh * hkv * per_tok_int2
        b += min(L, 144) * hkv * 2 * 256
        b += ((nh + 15) // 16) * 4 + 9 * 4
    b += len(lens) * hq * HEAD_DIM * (2 + 4)
    b += 2 * 128 * 128 * 4
    return b


def attend_bytes(lens, hkv, G, bits=2):
    """Algorithmic bytes of the split-K attention kernel of one decode call:
    INT2 (or INT4) codes + fp16 meta of every history token, raw bf16
    sink/recent tokens and the page-table entries it follows."""
    per_tok_int2 = 2 * (16 * bits + 4 * (128 // G))
    b = 0
    for L in lens:
        nh = n_hist_tokens(L)
        b += nh * hkv * per_tok_int2 + min(L, 144) * hkv * 2 * 256 + ((nh + 15) // 16) * 4 + 9 * 4
    return b


def append_bytes(batch, hkv, G, bits=2):
    """Algorithmic bytes of one append call: the evicted ring token is read
    and written to history, the new token is read and stored raw, R_K and
    R_V (fp32) are read once."""
    per_tok_int2 = 16 * bits + 4 * (128 // G)
    return batch * hkv * 2 * (256 + per_tok_int2 + 256 + 256) + 2 * 128 * 128 * 4


def write_bytes(lens, hkv, G):
    """Algorithmic bytes of one prefill write call: every new token's K and V
    read once (bf16), history tokens written as INT2 codes + fp16 meta, sink /
    recent tokens written raw; and of its history kernel alone."""
    per_tok_int2 = 32 + 4 * (128 // G)
    hist = raw = 0
    for L in lens:
        nh = n_hist_tokens(L)
        hist += nh * hkv * 2 * (256 + per_tok_int2)
        raw += min(L, 144) * hkv * 2 * (256 + 256)
    return hist + raw, hist


def bf16_bytes(lens, hq, hkv):
    b = 0
    for L in lens:
        b += L * hkv * 2 * 256 + ((L + 15) // 16) * 4
    return b + len(lens) * hq * HEAD_DIM * (2 + 4)


def main():
    args = parse_args()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path runs on a single GPU; "
              f"requests, KV heads or context ranges would shard across GPUs, with one exchange of the "
              f"per-query-head partials to merge a context split)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_rotated_kv_oscar_amd as oscar
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}))
        return

    workload_default = args.workload is None
    if workload_default:
        args.workload = "bs1"
    W = dict(WORKLOADS[args.workload])
    if args.layers:
        W["layers"] = args.layers
    if args.workload == "write":
        print(json.dumps(write_main(args, W, dev)))
        return
    if args.workload == "extend":
        print(json.dumps(extend_main(args, W, dev)))
        return
    line = decode_main(args, W, dev, args.workload)
    if workload_default and not args.no_companion:
        # every other workload, one after another (each frees its memory
        # before the next starts), then the device's read ceilings
        import gc
        for name in ("bs64", "28x100k", "int4_28x100k", "write", "extend", "config0"):
            gc.collect()
            torch.cuda.empty_cache()
            a2 = argparse.Namespace(**vars(args))
            a2.workload = name
            W2 = dict(WORKLOADS[name])
            t0 = time.time()
            if name == "write":
                leg = write_main(a2, W2, dev)
            elif name == "extend":
                leg = extend_main(a2, W2, dev)
            else:
                leg = decode_main(a2, W2, dev, name)
            leg["leg_wall_s"] = round(time.time() - t0, 1)
            for k in ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "data"):
                leg.pop(k, None)
            line[name] = leg
            print(f"leg {name}: {leg['value']} {leg['unit']} ({leg['leg_wall_s']} s)", file=sys.stderr, flush=True)
        gc.collect()
        torch.cuda.empty_cache()
        ceil = read_ceiling(dev)
        line["read_ceiling"] = ceil
        attach_ceiling(line, ceil)
        for name in ("bs64", "28x100k", "int4_28x100k", "write", "config0"):
            attach_ceiling(line[name], ceil)
    elif args.workload != "config0":
        ceil = read_ceiling(dev)
        line["read_ceiling"] = ceil
        attach_ceiling(line, ceil)
    print(json.dumps(line))


# gather block of each workload's history pages, and which ceiling bounds it
CEILING_OF = {"bs1": "gather_1280", "bs64": "gather_1280", "28x100k": "gather_1152", "int4_28x100k": "gather_2176",
              "write": "stream"}


def read_ceiling(dev, reps=5):
    """Measured read ceilings (oscar_read_probe, median of `reps` timed
    launches): streaming 4 KB blocks of a 4 GiB buffer, and gathers of
    history-page-sized blocks (INT2: 1152 / 1280 / 1536 B for G = 128 / 64 /
    32; INT4 G = 128: 2176 B) in a seeded random order from a 4 GiB pool."""
    import numpy as np
    import torch

    import bit_rotated_kv_oscar_amd as oscar
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {"probe": "oscar_read_probe, 16-byte loads, median of %d launches" % reps}

    def timed(n_blocks, bb, ids=None):
        ts = []
        for r in range(reps + 1):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            a1.record()
            oscar.profile_events(a0, a1)
            oscar.read_probe(buf, n_blocks, bb, ids, sink)
            torch.cuda.synchronize()
            if r:
                ts.append(a0.elapsed_time(a1) * 1e-3)
        return n_blocks * bb / float(np.median(ts)) / 1e9

    out["stream"] = round(timed(nbytes // 4096, 4096), 1)
    for bb in (1152, 1280, 1536, 2176):
        n_slots = nbytes // bb
        ids = torch.from_numpy(np.random.default_rng(bb).permutation(n_slots)[: n_slots * 3 // 4].astype(np.int32))
        out[f"gather_{bb}"] = round(timed(ids.numel(), bb, ids.to(dev)), 1)
    out["unit"] = "GB/s"
    del buf
    return out


def attach_ceiling(leg, ceil):
    """Adds the measured ceiling that bounds a bandwidth-bound leg and its
    dominant kernel's fraction of it."""
    wl = None
    for k, v in WORKLOADS.items():
        if v["name"] == leg.get("config", {}).get("workload"):
            wl = k
    key = CEILING_OF.get(wl)
    r = leg.get("roofline")
    if key is None or not r or r.get("unit") != "GB/s":
        return
    r["measured_ceiling"] = {"kind": key, "GBps": ceil[key]}
    r["frac_of_measured_ceiling"] = round(r["achieved"] / ceil[key], 4)


def replay_stats(run_once, steps):
    """Times `steps` calls of run_once (one replay each) with an event after
    each: mean over the whole bracket, median, p10 and p90 of the single
    replays (ms)."""
    import numpy as np
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        run_once()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return {"mean": ev[0].elapsed_time(ev[-1]) / steps, "median": float(np.median(per)),
            "p10": float(np.percentile(per, 10)), "p90": float(np.percentile(per, 90))}


def stats_fields(st):
    return {"ms_per_step_median": round(st["median"], 4), "ms_per_step_p10": round(st["p10"], 4),
            "ms_per_step_p90": round(st["p90"], 4)}


def host_info(threads_used):
    """Cores the CPU baseline used, the host's logical CPUs and CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cores": int(threads_used), "nproc": int(avail), "cpu_count": int(os.cpu_count() or 0),
            "cpu_model": model}


def blas_threads():
    try:
        import threadpoolctl
        return max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def decode_main(args, W, dev, workload):
    """A decode workload: per-layer caches prefilled, then graph-replayed
    steps of write-on-append + decode; returns the bench line."""
    import numpy as np
    import torch

    import bit_rotated_kv_oscar_amd as oscar
    import synth

    if args.layers:
        W["layers"] = args.layers
    nl, hq, hkv, G, B = W["layers"], W["hq"], W["hkv"], W["G"], W["batch"]
    bits = W.get("bits", 2)
    steps, warm = args.steps, args.warmup
    headroom = steps + warm + 1
    if W["batch"] == 1:
        final_lens = np.array([W["len_hi"]], dtype=np.int32)
    else:
        final_lens = synth.request_lengths(args.seed, B, W["len_lo"], W["len_hi"])
    start_lens = final_lens - headroom          # prefill length; each step appends one token
    max_len = int(final_lens.max())
    t_setup = time.time()

    # ---------------------------------------------------------------- layers
    class Layer:
        pass

    layers = []
    bf16_layers = []
    pages_per_req = [synth.hist_pages_needed(int(L)) for L in final_lens]
    bulk = None
    if "bf16_bytes_note" in W:
        # the capacity workloads draw every layer's prefill tokens into the
        # same buffers (per-layer allocations of ~17 GB between the pools
        # fragment the caching allocator)
        nel = int(start_lens.sum()) * hkv * HEAD_DIM
        bulk = (torch.empty(nel, dtype=torch.bfloat16, device=dev), torch.empty(nel, dtype=torch.bfloat16, device=dev),
                torch.empty(nel, dtype=torch.float32, device=dev))
    for l in range(nl):
        ly = Layer()
        ld = synth.LayerData(args.seed, l, hq, hkv)
        # calibration on the device (library), 2048 seeded tokens
        g = synth.device_generator(args.seed, l, synth.S_CAL_Q)
        qc = synth.q_device(g, 2048, hq, ld.lam, dev)
        kc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_K), 2048, ld.outliers, dev)
        vc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_V), 2048, ld.outliers, dev)
        R_K, R_V, ck, cv = oscar.calibrate_rotation(qc, kc, vc, 0.999)
        ly.rk, ly.rv = oscar.Rotation(R_K, ck, dev), oscar.Rotation(R_V, cv, dev)
        # page tables: every request's history pages from one shuffled pool
        if W.get("contiguous_pages"):
            hist_pt = np.arange(sum(pages_per_req), dtype=np.int32).reshape(B, -1)
            n_pool = sum(pages_per_req)
            bf16_pt = synth.bf16_page_tables(B)
        else:
            hist_pt, n_pool = synth.shuffled_page_tables(args.seed, l, final_lens,
                                                         n_pool_pages=sum(pages_per_req) + 1)
            bf16_pt = synth.bf16_page_tables(B, shuffle_seed=args.seed + l)
        ly.cache = oscar.LayerCache(hkv, G, n_pool, 9 * B, torch.from_numpy(hist_pt), torch.from_numpy(bf16_pt),
                                    device=dev, code_bits=bits)
        # prefill: every request's first start_len tokens in one write call
        tot = int(start_lens.sum())
        kw = dict(out=bulk[0], work=bulk[2]) if bulk else {}
        vw = dict(out=bulk[1], work=bulk[2]) if bulk else {}
        k = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CACHE_K), tot, ld.outliers, dev, **kw)
        v = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CACHE_V), tot, ld.outliers, dev, **vw)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(start_lens)]).astype(np.int32)).to(dev)
        oscar.write_kv(ly.cache, ly.rk, ly.rv, k, v, cu, torch.zeros(B, dtype=torch.int32, device=dev),
                       int(start_lens.max()))
        if bulk:
            torch.cuda.synchronize()   # the write has read the bulk tokens before the next layer redraws them
        # per-step inputs (the same new token and query every step)
        ly.k_new = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_K), B, ld.outliers, dev)
        ly.v_new = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_V), B, ld.outliers, dev)
        ly.q = synth.q_device(synth.device_generator(args.seed, l, synth.S_DEC_Q), B, hq, ld.lam, dev)
        ly.out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
        ly.ws = torch.zeros(oscar.decode_workspace_bytes(B, hq, hkv, max_len), dtype=torch.uint8, device=dev)
        layers.append(ly)
        if not args.no_bf16 and "bf16_bytes_note" not in W:
            # the same tokens, all raw bf16, for the in-run BF16 baseline
            bl = Layer()
            n_pages = [(int(L) + 15) // 16 for L in final_lens]
            pt, npg = synth.shuffled_page_tables(args.seed + 100, l, final_lens, n_pool_pages=sum(n_pages),
                                                 n_pages_fn=lambda L: (L + 15) // 16)
            kv = torch.zeros((npg, hkv, 2, 16, HEAD_DIM), dtype=torch.bfloat16, device=dev)
            ptd = torch.from_numpy(pt).to(dev)
            off = 0
            for bb in range(B):
                Ls = int(start_lens[bb])
                pos = torch.arange(Ls, device=dev)
                pg = ptd[bb, pos // 16]
                kv[pg, :, 0, pos % 16] = k[off:off + Ls]
                kv[pg, :, 1, pos % 16] = v[off:off + Ls]
                off += Ls
            bl.kv, bl.pt = kv, ptd
            bl.out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
            bl.ws = torch.zeros(oscar.bf16_decode_workspace_bytes(B, hq, hkv, max_len), dtype=torch.uint8,
                                device=dev)
            bf16_layers.append(bl)
        del k, v, qc, kc, vc
        if (l + 1) % 6 == 0 or l + 1 == nl:
            torch.cuda.synchronize()
            print(f"setup: {l + 1}/{nl} layers calibrated and prefilled ({time.time() - t_setup:.0f} s)",
                  file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    bulk = None
    torch.cuda.empty_cache()
    for ly in layers:
        assert int(ly.cache.status.item()) == 0, "prefill flagged bad data"
    setup_s = time.time() - t_setup

    # ---------------------------------------------------------------- the step
    lens_before = torch.from_numpy(start_lens.astype(np.int32)).to(dev)   # before this step's append
    lens_after = lens_before + 1

    def step():
        for ly in layers:
            oscar.decode_step(ly.cache, ly.rk, ly.rv, ly.k_new, ly.v_new, lens_before, ly.q, max_len,
                              1 / math.sqrt(HEAD_DIM), out=ly.out, workspace=ly.ws)
        lens_before.add_(1)
        lens_after.add_(1)

    def bf16_step():
        for bl in bf16_layers:
            oscar.bf16_paged_decode(layers[0].q, bl.kv, bl.pt, lens_after, max_len, 1 / math.sqrt(HEAD_DIM),
                                    out=bl.out, workspace=bl.ws)

    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    # one eager step checks that the launches work before capture; then rewind
    with torch.cuda.stream(stream):
        step()
        lens_before.sub_(1)
        lens_after.sub_(1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    # capture advanced nothing on the device; replays advance the lengths
    torch.cuda.synchronize()

    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    lens_at_timing = lens_before.cpu().numpy().copy()
    st = replay_stats(graph.replay, steps)
    ms_per_step = st["mean"]
    for ly in layers:
        assert int(ly.cache.status.item()) == 0, "decode flagged bad data"
        assert torch.isfinite(ly.out).all(), "non-finite decode output"

    # bytes per step, averaged over the timed steps (lengths grow by one per step)
    step_bytes = 0.0
    dec_bytes_mean = 0.0
    for s in range(steps):
        lens_s = (lens_at_timing + s + 1).tolist()
        db = decode_bytes(lens_s, hq, hkv, G, bits)
        dec_bytes_mean += db / steps
        step_bytes += nl * (db + append_bytes(B, hkv, G, bits)) / steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = B / (ms_per_step * 1e-3)

    # ------------------------------------------------ dominant-kernel timing
    # The split-K attention kernel dominates the step.  The library records a
    # pair of HIP events on the decode stream right around that one kernel
    # (oscar_profile_events); eager decode calls of every layer, three rounds.
    # A bounded spin kernel goes first, so that the calls queue up behind it
    # and run back to back, as in the replayed step (otherwise the device
    # idles between short kernels while the host issues the next call).
    pairs = []
    with torch.cuda.stream(stream):
        torch.cuda._sleep(20_000_000)
        for rep in range(3):
            for ly in layers:
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)   # creates the events; the library records them again
                a1.record(stream)
                oscar.profile_events(a0, a1)
                oscar.decode_attn(ly.cache, ly.rk, ly.rv, ly.q, lens_before, max_len, 1 / math.sqrt(HEAD_DIM),
                                  out=ly.out, workspace=ly.ws)
                pairs.append((a0, a1))
    torch.cuda.synchronize()
    attend_us = float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3
    lens_now0 = lens_before.cpu().numpy().tolist()
    attend_b = attend_bytes(lens_now0, hkv, G, bits)
    achieved = attend_b / (attend_us * 1e-6) / 1e9

    # ---------------------------------------------------------------- BF16
    bf16 = None
    if bf16_layers:
        lens_after.copy_(lens_before)   # decode the same lengths
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            bf16_step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g2, stream=stream):
            bf16_step()
        torch.cuda.synchronize()
        for _ in range(max(2, warm)):
            g2.replay()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(steps):
            g2.replay()
        b1.record()
        torch.cuda.synchronize()
        bf16_ms = b0.elapsed_time(b1) / steps
        # INT2 decode-only graph over the same lengths, for the like-for-like ratio
        g3 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g3, stream=stream):
            for ly in layers:
                oscar.decode_attn(ly.cache, ly.rk, ly.rv, ly.q, lens_after, max_len, 1 / math.sqrt(HEAD_DIM),
                                  out=ly.out, workspace=ly.ws)
        torch.cuda.synchronize()
        for _ in range(max(2, warm)):
            g3.replay()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(steps):
            g3.replay()
        c1.record()
        torch.cuda.synchronize()
        int2_dec_ms = c0.elapsed_time(c1) / steps
        lens_now = lens_before.cpu().numpy().tolist()
        bf16 = {"bf16_ms_per_step": round(bf16_ms, 4), "int2_decode_ms_per_step": round(int2_dec_ms, 4),
                "int2_speedup_vs_bf16": round(bf16_ms / int2_dec_ms, 3),
                "bf16_GBps": round(nl * bf16_bytes(lens_now, hq, hkv) / (bf16_ms * 1e-3) / 1e9, 1)}

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        # 28 x 100K: one KV head (with its query heads) of one request per
        # layer sample; the others: every head
        cpu = cpu_baseline(args, W, final_lens, step_bytes, kv_sample=1 if W["hkv"] * W["len_hi"] > 400000 else None,
                           bits=bits)

    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": W["name"], "layers": nl, "batch": B, "q_heads": hq, "kv_heads": hkv, "group": G,
                   "context": int(max_len) if B == 1 else [int(W["len_lo"]), int(W["len_hi"])],
                   "code_bits": bits,
                   "step": f"per layer: oscar_decode_step (write-on-append of one token + INT{bits} paged decode)"},
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(workload),
                     "kernel": f"oscar::attend_kernel<{hq // hkv}, {128 // G}> (split-K INT{bits} + BF16 decode)",
                     "avg_launch_us": round(attend_us, 2), "bytes_per_launch": int(attend_b)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    line.update(stats_fields(st))
    if bf16:
        line.update(bf16)
    elif "bf16_bytes_note" in W:
        line["bf16_baseline"] = "not run: " + W["bf16_bytes_note"]
    return line

def write_main(args, W, dev):
    """The write workload: 36 layers' prefill of 8 x 32768 tokens per step,
    then 64 append + decode steps (one HIP graph per step)."""
    import numpy as np
    import torch

    import bit_rotated_kv_oscar_amd as oscar
    import synth

    nl, hq, hkv, G, B = W["layers"], W["hq"], W["hkv"], W["G"], W["batch"]
    L = int(W["len_hi"])
    steps, warm = args.steps, args.warmup
    n_dec = 64
    lens = np.full(B, L, dtype=np.int32)
    t_setup = time.time()
    # the prompts (shared by every layer: inputs resident in HBM)
    ld0 = synth.LayerData(args.seed, 0, hq, hkv)
    k = synth.kv_device(synth.device_generator(args.seed, 0, synth.S_CACHE_K), B * L, ld0.outliers, dev)
    v = synth.kv_device(synth.device_generator(args.seed, 0, synth.S_CACHE_V), B * L, ld0.outliers, dev)
    cu = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * L).to(dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)

    class Layer:
        pass

    layers = []
    final = lens + n_dec + 1
    for l in range(nl):
        ly = Layer()
        ld = synth.LayerData(args.seed, l, hq, hkv)
        qc = synth.q_device(synth.device_generator(args.seed, l, synth.S_CAL_Q), 2048, hq, ld.lam, dev)
        kc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_K), 2048, ld.outliers, dev)
        vc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_V), 2048, ld.outliers, dev)
        R_K, R_V, ck, cv = oscar.calibrate_rotation(qc, kc, vc, 0.999)
        ly.rk, ly.rv = oscar.Rotation(R_K, ck, dev), oscar.Rotation(R_V, cv, dev)
        pages = [synth.hist_pages_needed(int(x)) for x in final]
        hist_pt, n_pool = synth.shuffled_page_tables(args.seed, l, final, n_pool_pages=sum(pages) + 1)
        ly.cache = oscar.LayerCache(hkv, G, n_pool, 9 * B, torch.from_numpy(hist_pt),
                                    torch.from_numpy(synth.bf16_page_tables(B, shuffle_seed=args.seed + l)),
                                    device=dev)
        ly.k_new = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_K), B, ld.outliers, dev)
        ly.v_new = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_V), B, ld.outliers, dev)
        ly.q = synth.q_device(synth.device_generator(args.seed, l, synth.S_DEC_Q), B, hq, ld.lam, dev)
        ly.out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=dev)
        ly.ws = torch.zeros(oscar.decode_workspace_bytes(B, hq, hkv, int(final.max())), dtype=torch.uint8,
                            device=dev)
        layers.append(ly)
        del qc, kc, vc
        if (l + 1) % 6 == 0 or l + 1 == nl:
            torch.cuda.synchronize()
            print(f"setup: {l + 1}/{nl} layers calibrated ({time.time() - t_setup:.0f} s)", file=sys.stderr,
                  flush=True)
    setup_s = time.time() - t_setup

    def prefill():
        for ly in layers:
            oscar.write_kv(ly.cache, ly.rk, ly.rv, k, v, cu, zeros, L)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            prefill()
        torch.cuda.synchronize()
        st = replay_stats(prefill, steps)
        ms_per_step = st["mean"]
        # dominant kernel: the history write kernel of each layer's call
        pairs = []
        for ly in layers:
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            a1.record(stream)
            oscar.profile_events(a0, a1)
            oscar.write_kv(ly.cache, ly.rk, ly.rv, k, v, cu, zeros, L)
            pairs.append((a0, a1))
        torch.cuda.synchronize()
    for ly in layers:
        assert int(ly.cache.status.item()) == 0, "write flagged bad data"
    hist_us = float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3
    all_b, hist_b = write_bytes(lens.tolist(), hkv, G)
    gbs = nl * all_b / (ms_per_step * 1e-3) / 1e9
    achieved = hist_b / (hist_us * 1e-6) / 1e9

    # 64 decode steps, each the write-on-append of one token + INT2 decode
    lens_before = torch.from_numpy(lens.copy()).to(dev)
    scale = 1 / math.sqrt(HEAD_DIM)
    max_len = int(final.max())

    def dstep():
        for ly in layers:
            oscar.decode_step(ly.cache, ly.rk, ly.rv, ly.k_new, ly.v_new, lens_before, ly.q, max_len, scale,
                              out=ly.out, workspace=ly.ws)
        lens_before.add_(1)

    with torch.cuda.stream(stream):
        dstep()
        lens_before.sub_(1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        dstep()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(n_dec):
        graph.replay()
    d1.record()
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / n_dec
    for ly in layers:
        assert int(ly.cache.status.item()) == 0, "decode flagged bad data"
        assert torch.isfinite(ly.out).all(), "non-finite decode output"

    cpu = None if args.no_cpu_baseline else write_cpu_baseline(args, W, all_b / (B * L))
    line = {
        "metric": WRITE_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": W["name"], "layers": nl, "batch": B, "q_heads": hq, "kv_heads": hkv, "group": G,
                   "new_tokens_per_prompt": L,
                   "step": "per layer: oscar_write_kv of every prompt (history rotated on the matrix cores, "
                           "clipped, INT2-packed; sink and recent raw)"},
        "tokens_per_s": round(B * L / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("write"),
                     "kernel": f"oscar::write_hist_kernel<{G}> (rotate, clip, INT2-pack, page-store)",
                     "avg_launch_us": round(hist_us, 2), "bytes_per_launch": int(hist_b)},
        "append_decode": {"steps": n_dec, "ms_per_step": round(dec_ms, 4),
                          "tokens_per_s": round(B / (dec_ms * 1e-3), 1)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    line.update(stats_fields(st))
    return line


def extend_flops(prefix, chunk, hq):
    """Algorithmic flops of one extend call: every new token i of a request
    scores and weights prefix + i + 1 keys per query head (2 flops per
    multiply-add, QK^T and PV)."""
    return sum(hq * 4 * HEAD_DIM * (n * L0 + n * (n + 1) // 2) for L0, n in zip(prefix, chunk))


def extend_main(args, W, dev):
    """The extend workload: per layer, the new chunk of every request attends
    to its cached prefix (sink + INT2 history + recent window) and causally to
    itself.  The prefix caches are written once (untimed)."""
    import numpy as np
    import torch

    import bit_rotated_kv_oscar_amd as oscar
    import synth

    nl, hq, hkv, G, B = W["layers"], W["hq"], W["hkv"], W["G"], W["batch"]
    L0, n = int(W["len_hi"]), int(W["chunk"])
    steps, warm = args.steps, args.warmup
    t_setup = time.time()
    prefix = np.full(B, L0, dtype=np.int32)
    cu = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * n).to(dev)
    lb = torch.from_numpy(prefix).to(dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)
    cu_pre = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * L0).to(dev)

    class Layer:
        pass

    layers = []
    for l in range(nl):
        ly = Layer()
        ld = synth.LayerData(args.seed, l, hq, hkv)
        qc = synth.q_device(synth.device_generator(args.seed, l, synth.S_CAL_Q), 2048, hq, ld.lam, dev)
        kc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_K), 2048, ld.outliers, dev)
        vc = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CAL_V), 2048, ld.outliers, dev)
        R_K, R_V, ck, cv = oscar.calibrate_rotation(qc, kc, vc, 0.999)
        ly.rk, ly.rv = oscar.Rotation(R_K, ck, dev), oscar.Rotation(R_V, cv, dev)
        full = prefix + n
        pages = [synth.hist_pages_needed(int(x)) for x in full]
        hist_pt, n_pool = synth.shuffled_page_tables(args.seed, l, full, n_pool_pages=sum(pages) + 1)
        ly.cache = oscar.LayerCache(hkv, G, n_pool, 9 * B, torch.from_numpy(hist_pt),
                                    torch.from_numpy(synth.bf16_page_tables(B, shuffle_seed=args.seed + l)),
                                    device=dev)
        kp = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CACHE_K), B * L0, ld.outliers, dev)
        vp = synth.kv_device(synth.device_generator(args.seed, l, synth.S_CACHE_V), B * L0, ld.outliers, dev)
        oscar.write_kv(ly.cache, ly.rk, ly.rv, kp, vp, cu_pre, zeros, L0)
        ly.k = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_K), B * n, ld.outliers, dev)
        ly.v = synth.kv_device(synth.device_generator(args.seed, l, synth.S_NEW_V), B * n, ld.outliers, dev)
        ly.q = synth.q_device(synth.device_generator(args.seed, l, synth.S_DEC_Q), B * n, hq, ld.lam, dev)
        ly.out = torch.empty((B * n, hq, HEAD_DIM), dtype=torch.float32, device=dev)
        layers.append(ly)
        del qc, kc, vc, kp, vp
        if (l + 1) % 6 == 0 or l + 1 == nl:
            torch.cuda.synchronize()
            print(f"setup: {l + 1}/{nl} layers calibrated and prefilled ({time.time() - t_setup:.0f} s)",
                  file=sys.stderr, flush=True)
    setup_s = time.time() - t_setup
    scale = 1 / math.sqrt(HEAD_DIM)

    def step():
        for ly in layers:
            oscar.extend_attn(ly.cache, ly.rk, ly.rv, ly.q, ly.k, ly.v, cu, lb, n, L0, scale, out=ly.out)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            step()
        torch.cuda.synchronize()
        st = replay_stats(step, steps)
        ms_per_step = st["mean"]
        pairs = []
        for ly in layers:
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            a1.record(stream)
            oscar.profile_events(a0, a1)
            oscar.extend_attn(ly.cache, ly.rk, ly.rv, ly.q, ly.k, ly.v, cu, lb, n, L0, scale, out=ly.out)
            pairs.append((a0, a1))
        torch.cuda.synchronize()
    for ly in layers:
        assert int(ly.cache.status.item()) == 0, "extend flagged bad data"
        assert torch.isfinite(ly.out).all(), "non-finite extend output"
    kern_us = float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3
    fl = extend_flops(prefix.tolist(), [n] * B, hq)
    tflops = nl * fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (kern_us * 1e-6) / 1e12
    cpu = None if args.no_cpu_baseline else extend_cpu_baseline(args, W)
    line = {
        "metric": EXTEND_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": W["name"], "layers": nl, "batch": B, "q_heads": hq, "kv_heads": hkv, "group": G,
                   "prefix": L0, "chunk": n,
                   "step": "per layer: oscar_extend_attn of the chunk over the cached prefix (INT2 history "
                           "scored on exact codes against q R_K, BF16 sink / window / chunk raw, causal chunk)"},
        "tokens_per_s": round(B * n / (ms_per_step * 1e-3), 1),
        "pct_mfma_peak": round(100 * tflops / MFMA_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": measured_traffic("extend"),
                     "kernel": f"oscar::extend_kernel<4, {G}> (INT2 + BF16 extend attention)",
                     "avg_launch_us": round(kern_us, 2), "flops_per_launch": int(fl)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    line.update(stats_fields(st))
    return line


def extend_cpu_baseline(args, W):
    """The fp64 oracle's extend timed on the host on a bounded sample: one
    layer, one request, the first 8 tokens of the chunk over the full prefix
    (the prefix written untimed); reported in algorithmic TFLOP/s."""
    import numpy as np

    import synth
    from oracle import oscar_ref as o
    threads = blas_threads()
    hq, hkv, G = W["hq"], W["hkv"], W["G"]
    L0, m = int(W["len_hi"]), 8
    ld = synth.LayerData(args.seed + 1000, 0, hq, hkv)
    k, v = ld.cache_kv(L0 + m)
    R = np.linalg.qr(np.random.default_rng(args.seed).standard_normal((128, 128)))[0]
    pt, npool = synth.shuffled_page_tables(args.seed, 0, [L0 + m])
    ref = o.LayerCacheRef(hkv, G, npool, 9, pt, synth.bf16_page_tables(1))
    ref.write(R, R, 6.0, 6.0, k[:L0], v[:L0], [0, L0], [0])
    q = ld.decode_q(m)
    t0 = time.time()
    o.extend_attn(ref, R, R, q, k[L0:], v[L0:], [0, m], [L0], 1 / math.sqrt(HEAD_DIM))
    dt = time.time() - t0
    fl = extend_flops([L0], [m], hq)
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
           "sample": f"first {m} chunk tokens of one request over its {L0}-token prefix, one layer (Hq {hq}, "
                     f"Hkv {hkv}, G {G}): {dt:.1f} s, {m / dt:.2f} tokens/s"}
    out.update(host_info(threads))
    return out


def write_cpu_baseline(args, W, bytes_per_token):
    """The fp64 oracle's write timed on the host on a bounded sample: one
    prompt of one layer written in chunks of 1024 tokens for about 15 s;
    scaled by the algorithmic bytes per token of the whole step."""
    import numpy as np

    import synth
    from oracle import oscar_ref as o
    threads = blas_threads()
    hq, hkv, G = W["hq"], W["hkv"], W["G"]
    L = int(W["len_hi"])
    ld = synth.LayerData(args.seed + 1000, 0, hq, hkv)
    k, v = ld.cache_kv(L)
    R = np.linalg.qr(np.random.default_rng(args.seed).standard_normal((128, 128)))[0]
    pt, npool = synth.shuffled_page_tables(args.seed, 0, [L])
    ref = o.LayerCacheRef(hkv, G, npool, 9, pt, synth.bf16_page_tables(1))
    chunk, done = 1024, 0
    t0 = time.time()
    while done + chunk <= L and (done < 2 * chunk or time.time() - t0 < 15.0):
        ref.write(R, R, 6.0, 6.0, k[done:done + chunk], v[done:done + chunk], [0, chunk], [done])
        done += chunk
    tok_s = done / (time.time() - t0)
    out = {"value": round(tok_s * bytes_per_token / 1e9, 4), "unit": "GB/s", "kind": "oracle",
           "sample": f"first {done} tokens of one {L}-token prompt into one layer (Hkv {hkv}, G {G}), written in "
                     f"chunks of {chunk}: {tok_s:.0f} tokens/s x the bytes per token of one layer's write"}
    out.update(host_info(threads))
    return out


def cpu_baseline(args, W, final_lens, step_bytes, kv_sample=None, bits=2):
    """The fp64 oracle timed on the host on a bounded sample of the step: one
    layer of the first request (kv_sample: only that many KV heads, with their
    query heads), prefilled untimed, then rounds of (append one token +
    decode) timed for up to ~20 s.  value = the algorithmic bytes of the
    sampled rounds / their time, the same unit as the GPU's value; the whole
    step's time at that rate is reported as extrapolated."""
    import numpy as np

    import synth
    from oracle import oscar_ref as o
    threads = blas_threads()
    hq, hkv, G = W["hq"], W["hkv"], W["G"]
    gqa = hq // hkv
    hkv_s = kv_sample or hkv
    hq_s = gqa * hkv_s
    L = int(final_lens[0])
    ld = synth.LayerData(args.seed + 1000, 0, hq_s, hkv_s)
    k, v = ld.cache_kv(L + 16)
    rng = np.random.default_rng(args.seed)
    R = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    pt, npool = synth.shuffled_page_tables(args.seed, 0, [L + 16])
    ref = o.LayerCacheRef(hkv_s, G, npool, 9, pt, synth.bf16_page_tables(1), bits=bits)
    t_pre = time.time()
    ref.write(R, R, 6.0, 6.0, k[:L - 8], v[:L - 8], [0, L - 8], [0])
    prefill_s = time.time() - t_pre
    q = ld.decode_q(1)
    t0 = time.time()
    rounds, sample_bytes = 0, 0
    cur = L - 8
    while rounds < 8 and (rounds < 2 or time.time() - t0 < 20.0):
        ref.write(R, R, 6.0, 6.0, k[cur:cur + 1], v[cur:cur + 1], [0, 1], [cur])
        cur += 1
        o.decode_attn(ref, R, R, q, [cur], 1 / math.sqrt(128))
        sample_bytes += decode_bytes([cur], hq_s, hkv_s, G, bits) + append_bytes(1, hkv_s, G, bits)
        rounds += 1
    dt = time.time() - t0
    rate = sample_bytes / dt
    heads = f"{hkv_s} of {hkv} KV heads" if hkv_s != hkv else f"all {hkv} KV heads"
    exact = W["layers"] == 1 and len(final_lens) == 1 and hkv_s == hkv
    out = {"value": round(rate / 1e9, 4), "unit": "GB/s", "kind": "oracle",
           "sample": f"{rounds} rounds of (append 1 token + decode) on one layer of one {L}-token request "
                     f"({heads}, {gqa} query heads each, G {G}, INT{bits}): {dt / rounds:.2f} s per round; value = "
                     f"algorithmic bytes of those rounds / their time",
           "measured" if exact else "s_per_step_extrapolated": round(step_bytes / rate, 3),
           "prefill_untimed_s": round(prefill_s, 1)}
    out.update(host_info(threads))
    return out


if __name__ == "__main__":
    main()
