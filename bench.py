#!/usr/bin/env python3
"""Benchmark: one MLA decode step (absorb_q -> append_cache -> decode -> out_proj)
on synthetic DeepSeek-V3-shaped inputs on one MI355X.

Prints ONE JSON line on stdout.  ``value`` = cached-token reads per second over
the whole step (one read = one 576-value latent row consumed by all 128 heads of
one query token), inputs resident in HBM.  The ``roofline`` object covers the
decode call (the dominant kernel) with its algorithmic bytes, timed live with
HIP events on the library's stream; ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload batch64]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode: cached-token reads/s, % of HBM & bf16 MFMA roofline (V3 shapes)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "head_latent_attention_05_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def kv_reads(inp) -> int:
    """Sum over query tokens of the rows each attends."""
    tot = 0
    for b in range(len(inp.kv_lens)):
        L, q = int(inp.kv_lens[b]), int(inp.q_lens[b])
        if inp.workload.causal:
            tot += sum(L - q + j + 1 for j in range(q))
        else:
            tot += q * L
    return tot


def traffic_from_counters(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    if not os.path.exists(COUNTERS):
        return None
    try:
        c = json.load(open(COUNTERS))
        e = c.get(workload)
        if not e or e.get("source_sha") != source_hash():
            return None
        return e["traffic_bytes"]
    except Exception:
        return None


def cpu_baseline(workload: str, budget_s: float):
    """The oracle (cache append + naive explicit-decompression attention, fp64)
    on the first sequences of the workload, 16 heads at a time, until ~budget_s
    of CPU work.  Reads done are counted per head: one cached-token read is one
    row consumed by all heads, so k of H heads count k/H of it."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from head_latent_attention_05_amd import synth
    from oracle import mla_oracle as O

    full = synth.make_inputs(workload)
    wl, d = full.workload, full.dims
    H = d.num_heads
    lens = [int(x) for x in full.kv_lens]
    reads, spent, nseq, nheads = 0.0, 0.0, 0, 0
    for b, L in enumerate(lens):
        inp = synth.make_inputs(wl, kv_lens=[L], seed=1000 + b)
        t0 = time.perf_counter()
        pool = O.build_pool(inp, 64)
        spent += time.perf_counter() - t0
        rows = lambda i: O.gather_rows(pool, d, 64, inp.block_table, i, int(inp.kv_lens[i]))
        nseq += 1
        for h0 in range(0, H, 16):
            heads = list(range(h0, min(H, h0 + 16)))
            t0 = time.perf_counter()
            O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope, inp.q_pe, rows, inp.kv_lens,
                        inp.q_start, wl.causal, heads)
            spent += time.perf_counter() - t0
            reads += kv_reads(inp) * len(heads) / H
            nheads += len(heads)
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": reads / spent, "unit": "cached-token reads/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{nseq} of {len(lens)} sequences of '{workload}' (kv_len {lens[:nseq]}), "
                      f"{nheads} of their {nseq * H} (sequence, head) pairs, cache append + "
                      f"naive fp64 attention, {spent:.1f} s wall"}


COPY_BYTES = 1 << 30


def profile_decode(st, copies: int, calls: int) -> int:
    """Kernel launches for hardware-counter runs: a plain device-to-device copy
    of COPY_BYTES (its FETCH_SIZE / WRITE_SIZE per byte scale the decode
    kernel's counters to bytes), then `calls` decode calls rotating over the
    same cache copies as the timed benchmark."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=st.dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for i in range(calls):
        st.decode(st.pools[i % copies])
    torch.cuda.synchronize()
    log(f"[bench] profile mode: 1 copy of {COPY_BYTES} B, {calls} decode calls over {copies} "
        f"cache copies")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pool-copies", type=int, default=0,
                    help="cache copies rotated between steps (0: enough for >= 1 GB)")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="N",
                    help="counter-run mode: one 1 GiB device copy (the reference kernel for "
                         "scaling HBM byte counters), then N decode calls over the rotated "
                         "cache copies, nothing else; prints no JSON line")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (decode batches "
              "would shard by sequence with no exchange).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from head_latent_attention_05_amd import synth
    from head_latent_attention_05_amd.step import DeviceStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    inp = synth.make_inputs(args.workload)
    d = inp.dims
    reads = kv_reads(inp)
    pool_bytes = inp.num_blocks * 64 * d.row * (2 if d.dtype == "bf16" else 4)
    copies = args.pool_copies or max(1, min(8, -(-(1 << 30) // pool_bytes)))
    log(f"[bench] workload={args.workload} T={inp.T} kv_reads={reads} pool={pool_bytes/1e6:.1f} MB "
        f"x{copies}")
    st = DeviceStep(inp, pool_copies=copies)
    pools = st.pools
    if args.profile_decode:
        return profile_decode(st, copies, args.profile_decode)

    def step(i, ev=None):
        # ev: events before absorb / after absorb / after append / after decode / after out_proj
        p = pools[i % copies]
        if ev is not None:
            ev[0].record()
        st.absorb()
        if ev is not None:
            ev[1].record()
        st.append(p)
        if ev is not None:
            ev[2].record()
        st.decode(p)
        if ev is not None:
            ev[3].record()
        st.project()
        if ev is not None:
            ev[4].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i, evs[i])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps
    call_ms = {name: [ev[k].elapsed_time(ev[k + 1]) for ev in evs]
               for k, name in enumerate(["mla_absorb_q", "mla_append_cache", "mla_decode",
                                         "mla_out_proj"])}
    dec_ms = call_ms["mla_decode"]
    dec_avg = float(np.mean(dec_ms))
    log(f"[bench] step {ms*1e3:.1f} us (wall {wall/args.steps*1e6:.1f} us), decode avg "
        f"{dec_avg*1e3:.1f} us, p10 {np.percentile(dec_ms,10)*1e3:.1f} p90 "
        f"{np.percentile(dec_ms,90)*1e3:.1f}; " +
        ", ".join(f"{k} {np.mean(v)*1e3:.1f} us" for k, v in call_ms.items()))
    assert int(st.dev_error.item()) == 0

    esz = 2 if d.dtype == "bf16" else 4
    H, T = d.num_heads, inp.T
    dec_bytes = reads * d.row * esz + T * H * (d.row + d.d_latent) * esz
    # algorithmic bytes of the other calls: weights once plus activations in and out
    call_bytes = {
        "mla_absorb_q": (H * d.d_nope * d.d_latent + T * H * (d.d_nope + d.d_latent)) * esz,
        "mla_append_cache": T * (2 * d.row + 2 * H * d.d_rope) * esz,
        "mla_decode": dec_bytes,
        "mla_out_proj": (H * d.d_v * d.d_latent + T * H * d.d_latent) * esz + T * H * d.d_v * 4,
    }
    calls = {k: {"avg_us": float(np.mean(v)) * 1e3,
                 "p10_us": float(np.percentile(v, 10)) * 1e3,
                 "p50_us": float(np.percentile(v, 50)) * 1e3,
                 "p90_us": float(np.percentile(v, 90)) * 1e3,
                 "algorithmic_bytes": int(call_bytes[k]),
                 "gbs": call_bytes[k] / (float(np.mean(v)) * 1e-3) / 1e9}
             for k, v in call_ms.items()}
    dec_flops = reads * 2 * d.num_heads * (d.row + d.d_latent)
    achieved_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
    achieved_tfs = dec_flops / (dec_avg * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": reads / (ms * 1e-3),
        "unit": "cached-token reads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": int(len(inp.kv_lens)),
                   "query_tokens": inp.T, "kv_reads_per_step": reads,
                   "kv_len_min": int(inp.kv_lens.min()), "kv_len_max": int(inp.kv_lens.max()),
                   "heads": d.num_heads, "d_latent": d.d_latent, "d_rope": d.d_rope,
                   "block_size": 64, "causal": bool(inp.workload.causal),
                   "cache_copies_rotated": copies},
        "roofline": {"kernel": "mla_decode", "bound": "hbm", "achieved": achieved_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": traffic_from_counters(args.workload),
                     "algorithmic_bytes": dec_bytes, "avg_launch_us": dec_avg * 1e3,
                     "mfma": {"achieved": achieved_tfs, "peak": MFMA_BF16_PEAK_TFS,
                              "unit": "TFLOP/s", "frac": achieved_tfs / MFMA_BF16_PEAK_TFS,
                              "algorithmic_flops": dec_flops}},
        "calls": calls,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        rec["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
