#!/usr/bin/env python3
"""Benchmark: one MLA decode step (absorb_q -> append_cache -> decode -> out_proj)
on synthetic DeepSeek-V3-shaped inputs on one MI355X.

Prints ONE JSON line on stdout.  ``value`` = cached-token reads per second over
the whole step (one read = one 576-value latent row consumed by all 128 heads of
one query token), inputs resident in HBM.  The ``roofline`` object covers the
decode call (the dominant kernel) with its algorithmic bytes, timed live with
HIP events on the library's stream, against the HBM peak and against a 1 GiB
device copy timed in the same run; ``workloads`` gives the decode call alone on
the other workloads; ``cpu_baseline`` times the CPU oracle on a bounded sample
of the step's own inputs; ``fp8_cache`` repeats the step and the decode calls
with the e4m3 latent cache (576 bytes per cached token).

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
MFMA_FP8_PEAK_TFS = 5000.0   # MI355X dense fp8 MFMA
FP8_KV_SCALE = 2.0 ** -4     # e4m3 cache scale of the synthetic rows (magnitudes < ~6)
COUNTERS = os.path.join(ROOT, "profiles", "decode_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources of the decode call (its kernels, their launch and split plan): the
# committed counters stay valid while none of these changes.
DECODE_SOURCES = ("decode_v4.hip", "decode_fp8.hip", "tile_walk.h", "merge_v3.hip",
                  "plan_device.h", "gfx950_asm.h", "uniform_ptr.h", "mla_internal.h",
                  "mla_api.hip")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "head_latent_attention_05_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
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


def host_info():
    """Cores this process may run on and the CPU model name."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(inp, budget_s: float):
    """The oracle on the step's own inputs: with the history rows already in
    its cache (set-up, untimed, as on the GPU), it appends each sequence's new
    tokens and runs the naive explicit-decompression attention (fp64, up to the
    step's output) for that sequence, 16 heads at a time, until ~budget_s of
    CPU work.  Reads done are counted per head: one cached-token read is one row
    consumed by all heads, so k of H heads count k/H of it."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import mla_oracle as O

    wl, d = inp.workload, inp.dims
    H = d.num_heads
    cos32, sin32 = O.rope_table_f32(inp.max_pos(), d.d_rope)
    pool = O.build_pool(inp, 64, cos32, sin32, which="history")
    seqs, pos, ck, kp = inp.new_tokens()
    reads, spent, nseq, nheads = 0.0, 0.0, 0, 0
    for b in range(len(inp.kv_lens)):
        a0, a1 = int(inp.q_start[b]), int(inp.q_start[b + 1])
        t0 = time.perf_counter()
        O.append_cache(pool, d, 64, seqs[a0:a1], pos[a0:a1], ck[a0:a1], kp[a0:a1],
                       inp.block_table, cos32, sin32)
        spent += time.perf_counter() - t0
        L = int(inp.kv_lens[b])
        rows = lambda i, b=b, L=L: O.gather_rows(pool, d, 64, inp.block_table, b, L)
        q_start = np.array([0, a1 - a0], np.int64)
        nseq += 1
        for h0 in range(0, H, 16):
            heads = list(range(h0, min(H, h0 + 16)))
            t0 = time.perf_counter()
            O.naive_mla(d, inp.w_uk, inp.w_uv, inp.q_nope[a0:a1], inp.q_pe[a0:a1], rows,
                        np.array([L]), q_start, wl.causal, heads)
            spent += time.perf_counter() - t0
            q = a1 - a0
            r = sum(L - q + j + 1 for j in range(q)) if wl.causal else q * L
            reads += r * len(heads) / H
            nheads += len(heads)
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    host_cores, model = host_info()
    blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    lens = [int(x) for x in inp.kv_lens[:nseq]]
    return {"value": reads / spent, "unit": "cached-token reads/s",
            "cores": int(min(blas, host_cores)), "host_cores": host_cores, "cpu_model": model,
            "kind": "oracle",
            "sample": f"the timed step's own inputs: sequences 0..{nseq - 1} of "
                      f"{len(inp.kv_lens)} of '{wl.name}' (kv_len {lens}), {nheads} of their "
                      f"{nseq * H} (sequence, head) pairs; new-token cache append + naive fp64 "
                      f"attention to the step output, {spent:.1f} s wall"}


def copy_bandwidth(dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Device-to-device copy of nbytes (bytes read + bytes written) / time, in
    GB/s: the achievable streaming rate on this device, measured now."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def decode_bytes_flops(inp, fp8: bool = False):
    """Algorithmic bytes and flops of one decode call: every attended row read
    once per query token (1 byte per value for the e4m3 cache), q_lat read and
    o_lat written once; 2 flops per multiply-add over the 576-wide scores and
    the 512-wide values."""
    d = inp.dims
    esz = 2 if d.dtype == "bf16" else 4
    reads = kv_reads(inp)
    nbytes = reads * d.row * (1 if fp8 else esz) + inp.T * d.num_heads * (d.row + d.d_latent) * esz
    flops = reads * 2 * d.num_heads * (d.row + d.d_latent)
    return reads, nbytes, flops


def pool_copies_for(st, min_bytes: int = 1 << 30, cap: int = 256):
    """The step's cache plus clones of it, together at least min_bytes (so
    rotating over them keeps the working set far above the 256 MB Infinity
    Cache), at most cap copies."""
    nb = st.pool.numel() * st.pool.element_size()
    n = max(1, min(cap, -(-min_bytes // nb)))
    return [st.pool] + [st.pool.clone() for _ in range(n - 1)]


def decode_only(workload: str, calls: int, warmup: int, copy_gbs: float, kv_scale=None):
    """Decode-call time alone on another workload (same launch configuration as
    the headline step), over rotated cache copies; with kv_scale, over the e4m3
    cache (fp8 MFMA, rated against the fp8 peak)."""
    import numpy as np
    import torch

    from head_latent_attention_05_amd import synth
    from head_latent_attention_05_amd.step import DeviceStep

    inp = synth.make_inputs(workload)
    st = DeviceStep(inp, kv_scale=kv_scale)
    st.absorb()
    st.append()
    pools = pool_copies_for(st)
    torch.cuda.synchronize()
    for i in range(warmup):
        st.decode(pools[i % len(pools)])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        a.record()
        st.decode(pools[i % len(pools)])
        b.record()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    reads, nbytes, flops = decode_bytes_flops(inp, fp8=kv_scale is not None)
    gbs = nbytes / (avg * 1e-3) / 1e9
    tfs = flops / (avg * 1e-3) / 1e12
    peak_tfs = MFMA_FP8_PEAK_TFS if kv_scale is not None else MFMA_BF16_PEAK_TFS
    rec = {"decode_us": avg * 1e3, "p50_us": float(np.median(ms)) * 1e3, "calls": calls,
           "kv_reads": reads, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
           "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "copy_frac": gbs / copy_gbs,
           "mfma_tfs": tfs, "mfma_frac": tfs / peak_tfs, "mfma_peak_tfs": peak_tfs,
           "bound": "mfma" if inp.workload.causal and inp.T > len(inp.kv_lens) else "hbm",
           "cache_copies_rotated": len(pools)}
    if (inp.workload.causal and inp.T > len(inp.kv_lens) and inp.dims.dtype == "bf16"
            and kv_scale is None):
        rec["decompressed"] = decompressed_only(st, inp, pools, calls, reads)
    del st, pools
    torch.cuda.empty_cache()
    return rec


def upstream_calls(st, inp, calls: int, copy_gbs: float) -> dict:
    """Calls beyond the four of the step, on the same step's new tokens, each
    launch timed alone with HIP events; a 1 GiB read between launches (not
    timed) evicts the weights from L2 and the Infinity Cache, as the decode
    between two steps would.  (A fill would leave dirty lines whose write-back
    overlaps the timed call.)

    mla_kv_down_append: the joint KV down-projection of the new tokens' hidden
    states (d_model 7168, synthetic) with the latent RMSNorm, fused with the
    append.  Algorithmic bytes: the weight, the hidden states, the rows and the
    RoPE columns of q_lat written, the query RoPE inputs read.
    mla_absorb_q_fused / mla_out_proj_fused: the weight-level absorbed
    projections with synthetic fused weights (d_cq 1536, d_model 7168); bytes:
    the fused weight plus the activations in and out."""
    import numpy as np
    import torch

    from head_latent_attention_05_amd import binding as B
    from head_latent_attention_05_amd import synth
    from head_latent_attention_05_amd.step import to_device

    d = inp.dims
    esz = 2 if d.dtype == "bf16" else 4
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=st.dev)
    out = {}
    if d.dtype == "bf16" and d.num_heads == 128 and d.d_latent == 512 and d.d_rope == 64:
        d_model = 7168
        di = synth.make_down_inputs(d, inp.T, d_model, seed=41)
        up = lambda a: to_device(a, d.dtype, st.dev)
        x, w, b, g = up(di.x), up(di.w_dkv), up(di.b_dkv), up(di.gamma)
        ws = torch.empty(B.kv_down_workspace_size(st.cfg, inp.T, d_model), dtype=torch.uint8,
                         device=st.dev)

        def call():
            B.kv_down_append(st.cfg, x, w, b, g, di.eps, st.q_pe, st.new_seq, st.new_pos,
                             st.block_table, st.num_blocks, st.rope_cos, st.rope_sin, ws,
                             st.pool, st.q_lat, dev_error=st.dev_error)

        n = d.d_latent + d.d_rope
        nbytes = (n * d_model + inp.T * d_model + n + d.d_latent + inp.T * d.row
                  + 2 * inp.T * d.num_heads * d.d_rope) * esz
        ms = []
        for i in range(calls + 2):
            flush.sum()
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            e.record()
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(a.elapsed_time(e))
        assert int(st.dev_error.item()) == 0
        avg = float(np.mean(ms))
        gbs = nbytes / (avg * 1e-3) / 1e9
        out["mla_kv_down_append"] = {
            "avg_us": avg * 1e3, "p50_us": float(np.median(ms)) * 1e3, "calls": calls,
            "d_model": d_model, "tokens": inp.T, "algorithmic_bytes": int(nbytes),
            "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "copy_frac": gbs / copy_gbs,
            "bound": "hbm"}
        # weight-level absorption: the fused query-side and output-side weights
        d_cq = 1536
        fi = synth.make_fused_inputs(d, inp.T, d_cq, d_model, seed=42)
        c_q, w_kq = up(fi.c_q), up(fi.w_kq)
        o_lat, w_ov = up(fi.o_lat), up(fi.w_ov)
        q_lat = torch.empty_like(st.q_lat)
        out_f = torch.empty((inp.T, d_model), dtype=torch.float32, device=st.dev)
        ws_f = torch.empty(B.out_proj_fused_workspace_size(st.cfg, inp.T, d_model),
                           dtype=torch.uint8, device=st.dev)
        H, dc = d.num_heads, d.d_latent
        fused = {
            "mla_absorb_q_fused": (lambda: B.absorb_q_fused(st.cfg, c_q, w_kq, q_lat),
                                   (H * d_cq * dc + inp.T * d_cq + inp.T * H * dc) * esz,
                                   {"d_cq": d_cq}),
            "mla_out_proj_fused": (lambda: B.out_proj_fused(st.cfg, o_lat, w_ov, out_f, ws_f),
                                   (H * dc * d_model + inp.T * H * dc) * esz
                                   + inp.T * d_model * 4, {"d_model": d_model}),
        }
        for name, (fn, nb, extra) in fused.items():
            ms = []
            for i in range(calls + 2):
                flush.sum()
                a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                e.record()
                torch.cuda.synchronize()
                if i >= 2:
                    ms.append(a.elapsed_time(e))
            avg = float(np.mean(ms))
            gbs = nb / (avg * 1e-3) / 1e9
            out[name] = {"avg_us": avg * 1e3, "p50_us": float(np.median(ms)) * 1e3,
                         "calls": calls, "tokens": inp.T, "algorithmic_bytes": int(nb),
                         "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "copy_frac": gbs / copy_gbs,
                         "bound": "hbm", **extra}
        del c_q, w_kq, o_lat, w_ov, q_lat, out_f, ws_f
    del flush
    torch.cuda.empty_cache()
    return out


def decompressed_only(st, inp, pools, calls: int, pairs: int) -> dict:
    """The same prefill through mla_prefill_decompressed (explicit decompression
    of K and V, then attention at widths 192 / 128).  Algorithmic FLOPs: the
    decompression of every cached row of the batch for every head
    (2 * rows * d_c * (d_nope + d_v) * H) plus 2 * H * (d_nope + d_rope + d_v)
    per attended (query, key) pair."""
    import numpy as np
    import torch

    from head_latent_attention_05_amd import binding as B

    d = inp.dims
    ws = torch.empty(B.prefill_workspace_size(st.cfg, st.q_start_host, st.kv_lens_host),
                     dtype=torch.uint8, device=st.dev)
    out = torch.empty((inp.T, d.num_heads, d.d_v), dtype=torch.float32, device=st.dev)

    def call(pool):
        B.prefill_decompressed(st.cfg, st.q_start, st.kv_lens, st.q_start_host, st.kv_lens_host,
                               st.block_table, st.num_blocks, st.q_nope, st.q_lat, pool, st.w_uk,
                               st.w_uv, st.causal, ws, out, dev_error=st.dev_error)

    for i in range(2):
        call(pools[i % len(pools)])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        a.record()
        call(pools[i % len(pools)])
        b.record()
    torch.cuda.synchronize()
    assert int(st.dev_error.item()) == 0
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = float(np.mean(ms))
    rows = int(sum(-(-int(L) // 64) * 64 for L in inp.kv_lens))
    flops = (2 * rows * d.d_latent * (d.d_nope + d.d_v) * d.num_heads
             + 2 * d.num_heads * (d.d_nope + d.d_rope + d.d_v) * pairs)
    tfs = flops / (avg * 1e-3) / 1e12
    del ws, out
    return {"call_us": avg * 1e3, "p50_us": float(np.median(ms)) * 1e3, "calls": calls,
            "algorithmic_flops": int(flops), "mfma_tfs": tfs,
            "mfma_frac": tfs / MFMA_BF16_PEAK_TFS, "bound": "mfma"}


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


def _short_kernel(name: str) -> str:
    for pre in ("void ", "mla::(anonymous namespace)::"):
        name = name.replace(pre, "")
    return name.split("(")[0]


def read_counter_runs(dirs):
    """Mean value per dispatch of every (kernel, counter) in rocprofv3 --pmc CSV
    output directories; also the dispatch counts."""
    import csv
    import collections
    vals = collections.defaultdict(list)
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    vals[(_short_kernel(r["Kernel_Name"]), r["Counter_Name"])].append(
                        float(r["Counter_Value"]))
    return vals


DECODE_KERNELS = ("decode_v4_kernel", "decode_fp8_kernel", "merge_v3_kernel")


def counters_json(workload: str, dirs, out: str, fp8: bool = False) -> int:
    """From --pmc runs of `bench.py --profile-decode N` (FETCH_SIZE and
    WRITE_SIZE each in its own run): the 1 GiB copy's counters give KiB -> byte
    factors; the decode call's HBM bytes per launch are its kernels' scaled
    FETCH_SIZE + WRITE_SIZE.  Merged into `out`, keyed by workload and stamped
    with the kernel-source hash (bench.py ignores it once the sources change)."""
    vals = read_counter_runs(dirs)
    copy = [v for (k, c), v in vals.items() if "copyBuffer" in k and c == "FETCH_SIZE"]
    copyw = [v for (k, c), v in vals.items() if "copyBuffer" in k and c == "WRITE_SIZE"]
    if not copy or not copyw:
        log("no copy-kernel FETCH_SIZE / WRITE_SIZE found")
        return 1
    ff = COPY_BYTES / (max(max(v) for v in copy) * 1024)
    wf = COPY_BYTES / (max(max(v) for v in copyw) * 1024)
    per = {}
    for k in DECODE_KERNELS:
        fv, wv = vals.get((k, "FETCH_SIZE")), vals.get((k, "WRITE_SIZE"))
        if fv and wv:
            per[k] = {"fetch_bytes": sum(fv) / len(fv) * 1024 * ff,
                      "write_bytes": sum(wv) / len(wv) * 1024 * wf, "dispatches": len(fv)}
    if "decode_v4_kernel" not in per and "decode_fp8_kernel" not in per:
        log("no decode kernel counters found")
        return 1
    from head_latent_attention_05_amd import synth
    _, alg, _ = decode_bytes_flops(synth.make_inputs(workload), fp8=fp8)
    traffic = sum(v["fetch_bytes"] + v["write_bytes"] for v in per.values())
    rec = json.load(open(out)) if os.path.exists(out) else {}
    key = workload + ("_fp8" if fp8 else "")
    rec[key] = {"source_sha": source_hash(), "traffic_bytes": traffic,
                     "algorithmic_bytes": alg, "traffic_over_algorithmic": traffic / alg,
                     "fetch_factor": ff, "write_factor": wf, "kernels": per}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec[key], indent=1))
    return 0


def fp8_section(inp, args, copy_gbs: float, workloads) -> dict:
    """The step of the headline workload with the e4m3 cache (absorb ->
    fp8 append -> fp8 decode -> out_proj, timed as the bf16 step), then the fp8
    decode call alone on each workload."""
    import numpy as np
    import torch

    from head_latent_attention_05_amd.step import DeviceStep

    d = inp.dims
    reads = kv_reads(inp)
    pool_bytes = inp.num_blocks * 64 * d.row
    copies = max(1, min(16, -(-(1 << 30) // pool_bytes)))
    st = DeviceStep(inp, pool_copies=copies, kv_scale=FP8_KV_SCALE)

    def step(i):
        p = st.pools[i % copies]
        st.absorb()
        st.append(p)
        st.decode(p)
        st.project()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record()
    for i in range(args.steps):
        step(i)
    b_.record()
    torch.cuda.synchronize()
    ms = a_.elapsed_time(b_) / args.steps
    assert int(st.dev_error.item()) == 0
    out = {"kv_scale": FP8_KV_SCALE, "format": "OCP e4m3, one power-of-two scale per cache",
           "decode_traffic_bytes": traffic_from_counters(args.workload + "_fp8"),
           "step_us": ms * 1e3, "value": reads / (ms * 1e-3), "unit": "cached-token reads/s",
           "cache_copies_rotated": copies}
    log(f"[bench] fp8 cache step {ms*1e3:.1f} us")
    del st
    torch.cuda.empty_cache()
    out["workloads"] = {}
    for w in workloads:
        r = decode_only(w, args.extra_calls, 2, copy_gbs, kv_scale=FP8_KV_SCALE)
        out["workloads"][w] = r
        log(f"[bench]   fp8 {w}: {r['decode_us']:.1f} us, {r['hbm_frac']*100:.1f} % HBM, "
            f"{r['mfma_frac']*100:.1f} % fp8 MFMA")
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-workloads", default="single,long,prefill",
                    help="comma-separated workloads whose decode call is also timed alone "
                         "(reported under 'workloads'); empty for none")
    ap.add_argument("--extra-calls", type=int, default=10)
    ap.add_argument("--fp8-workloads", default="batch64,single,long,prefill",
                    help="workloads whose decode call is also timed over the e4m3 cache "
                         "(reported under 'fp8_cache'); empty for none")
    ap.add_argument("--pool-copies", type=int, default=0,
                    help="cache copies rotated between steps (0: enough for >= 1 GB)")
    ap.add_argument("--profile-decode", type=int, default=0, metavar="N",
                    help="counter-run mode: one 1 GiB device copy (the reference kernel for "
                         "scaling HBM byte counters), then N decode calls over the rotated "
                         "cache copies, nothing else; prints no JSON line")
    ap.add_argument("--fp8", action="store_true",
                    help="with --profile-decode / --counters-json: the e4m3 cache")
    ap.add_argument("--counters-json", nargs="+", metavar="DIR",
                    help="no GPU: fold rocprofv3 --pmc output directories of the "
                         "--profile-decode mode into profiles/decode_counters.json")
    args = ap.parse_args()
    if args.counters_json:
        return counters_json(args.workload, args.counters_json, COUNTERS, fp8=args.fp8)
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
    if args.profile_decode and args.fp8:
        copies = max(1, min(16, -(-(1 << 30) // (pool_bytes // 2))))
        st = DeviceStep(inp, pool_copies=copies, kv_scale=FP8_KV_SCALE)
        return profile_decode(st, copies, args.profile_decode)
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

    def timed(run, n):
        """Mean ms per step of n back-to-back steps, bracketed by synchronisations."""
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w_ = time.perf_counter()
        a_.record()
        for i in range(n):
            run(i)
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n, (time.perf_counter() - w_) / n

    for i in range(args.warmup):
        step(i)
    # The step: the four calls launched back to back, with no events between them.
    ms, wall = timed(step, args.steps)
    # Per-call breakdown: a separate eager pass with events between the calls
    # (the events themselves add small gaps, so the step above is timed without).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = {name: [ev[k].elapsed_time(ev[k + 1]) for ev in evs]
               for k, name in enumerate(["mla_absorb_q", "mla_append_cache", "mla_decode",
                                         "mla_out_proj"])}
    dec_ms = call_ms["mla_decode"]
    dec_avg = float(np.mean(dec_ms))
    log(f"[bench] step {ms*1e3:.1f} us (wall {wall*1e6:.1f} us); decode avg "
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
    _, dec_bytes2, dec_flops = decode_bytes_flops(inp)
    assert dec_bytes2 == dec_bytes
    copy_gbs = copy_bandwidth(st.dev)
    log(f"[bench] 1 GiB device copy: {copy_gbs:.0f} GB/s")
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
                     "vs_copy": {"copy_gbs": copy_gbs, "frac": achieved_gbs / copy_gbs,
                                 "copy": "1 GiB device-to-device torch copy, same run"},
                     "mfma": {"achieved": achieved_tfs, "peak": MFMA_BF16_PEAK_TFS,
                              "unit": "TFLOP/s", "frac": achieved_tfs / MFMA_BF16_PEAK_TFS,
                              "algorithmic_flops": dec_flops}},
        "calls": calls,
    }
    rec["upstream_calls"] = upstream_calls(st, inp, args.extra_calls, copy_gbs)
    for k, v in rec["upstream_calls"].items():
        log(f"[bench] {k}: {v['avg_us']:.1f} us, {v['hbm_frac']*100:.1f} % HBM")
    extras = [w for w in args.extra_workloads.split(",") if w and w != args.workload]
    fp8_work = [w for w in args.fp8_workloads.split(",") if w]
    del st, pools
    torch.cuda.empty_cache()
    if fp8_work and d.dtype == "bf16":
        rec["fp8_cache"] = fp8_section(inp, args, copy_gbs, fp8_work)
    if extras:
        rec["workloads"] = {}
        for w in extras:
            log(f"[bench] decode call alone on '{w}' ...")
            rec["workloads"][w] = decode_only(w, args.extra_calls, 2, copy_gbs)
            log(f"[bench]   {w}: {rec['workloads'][w]['decode_us']:.1f} us, "
                f"{rec['workloads'][w]['hbm_frac']*100:.1f} % HBM, "
                f"{rec['workloads'][w]['mfma_frac']*100:.1f} % MFMA")
            if "decompressed" in rec["workloads"][w]:
                dc = rec["workloads"][w]["decompressed"]
                log(f"[bench]   {w} non-absorbed: {dc['call_us']:.1f} us, "
                    f"{dc['mfma_frac']*100:.1f} % MFMA")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
