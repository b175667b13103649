#!/usr/bin/env python3
"""Benchmark of generalized paged attention on one MI355X.

A step is one pass of the whole hot path over one batch: pa_kv_write of the
batch's new K/V, then pa_attention.  Default workload: batched decode on a
Llama-2-13B-like layer (64 sequences, contexts U[128, 4096], 40 heads,
head_dim 128, fp16, 16-token blocks from a shuffled free list).

Prints ONE JSON line: the KV-read throughput (algorithmic bytes of the K/V
the step must read / step time), query tokens/s, the roofline of the
dominant kernel (pa_attention) timed with HIP events on the stream it runs
on, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn KV-read GB/s (% HBM peak) and query tokens/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # dense matrix-core peak
BOUND = {"c1": "hbm", "c2": "hbm", "c3": "hbm", "c4": "hbm", "c5": "mfma"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_14_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def work_figures(wl):
    """Algorithmic work of one step (host arithmetic on the workload's metadata)."""
    B, D, e = wl.block_size, wl.head_dim, 2
    Hkv, Hq = wl.num_kv_heads, wl.num_q_heads
    C = wl.context_lens.astype(np.int64)
    n = wl.query_lens
    slots = []
    for s in range(wl.num_seqs):
        j = np.arange(C[s])
        slots.append(wl.block_tables[s, j // B].astype(np.int64) * B + j % B)
    uniq = np.unique(np.concatenate(slots)).size if slots else 0
    per_token = Hkv * D * 2 * e                       # K and V of one token, all KV heads
    flops = int(np.sum(Hq * 4 * D * (n * (C - n) + n * (n + 1) // 2)))
    written = int((wl.slot_mapping >= 0).sum())
    return {
        "kv_bytes": int(uniq * per_token),             # unique visible (block, slot) K/V
        "kv_bytes_logical": int(C.sum() * per_token),
        "q_out_bytes": int(2 * wl.total_q * Hq * D * e),
        "kv_write_bytes": int(2 * written * per_token),  # read new rows + write pool rows
        "flops": flops,
        "query_tokens": int(wl.total_q),
    }


def attention_launches(wl):
    """The kernels one pa_attention call enqueues for this batch, in order (the
    library's dispatch rule restated from the host-visible sizes and lengths)."""
    G = wl.num_q_heads // wl.num_kv_heads
    rows = wl.query_lens * G
    names = []
    if G <= 8:  # sequences with at most 8 rows per KV head may exist
        if wl.num_seqs >= 2 and wl.max_context_len > 64:
            names += ["cascade_plan_kernel", "prefill_kernel<shared prefix>"]
        names.append("decode_kernel")
    if wl.max_query_len * G > 8:
        # calls with more than 128 query rows per KV head take the wide kernel
        # (its 8-wave form below 1024 rows)
        names.append("prefill_wide_kernel" if wl.max_query_len * G > 128 else "prefill_kernel")
    names.append(f"({int((rows <= 8).sum())} decode / {int((rows > 8).sum())} prefill sequences)")
    return names


def cpu_baseline(wl, target_s: float):
    """The oracle as it stands, on (sequence, KV head) pairs taken in order until
    about ``target_s`` seconds of CPU work; reported in the metric's unit."""
    from oracle import attention_ref, kv_write_ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    D, e = wl.head_dim, 2
    G = wl.num_q_heads // wl.num_kv_heads
    qsl = wl.query_start_loc
    spent, pairs, kv_bytes, row_heads = 0.0, 0, 0, 0
    done = False
    for s in range(wl.num_seqs):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        for g in range(wl.num_kv_heads):
            t0 = time.perf_counter()
            attention_ref(wl.q[lo:hi, g * G:(g + 1) * G], kp[:, g:g + 1], vp[:, g:g + 1],
                          wl.block_tables[s:s + 1], wl.context_lens[s:s + 1],
                          np.array([0, hi - lo], np.int32), 1, wl.scale, wl.dtype)
            spent += time.perf_counter() - t0
            pairs += 1
            kv_bytes += int(wl.context_lens[s]) * D * 2 * e
            row_heads += (hi - lo) * G
            if spent >= target_s:
                done = True
                break
        if done:
            break
    total_pairs = wl.num_seqs * wl.num_kv_heads
    return {
        "value": round(kv_bytes / spent / 1e9, 6),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on the first {pairs} of {total_pairs} (sequence, KV head) "
                   f"pairs: {row_heads} query rows x heads, {kv_bytes / 1e9:.3f} GB of K/V, "
                   f"{spent:.1f} s; BLAS threads {blas_threads}, "
                   f"{len(os.sched_getaffinity(0))} host cores visible"),
        "query_tokens_per_s": round(row_heads / wl.num_q_heads / spent, 3),
    }


def load_traffic(workload: str):
    """HBM bytes per pa_attention call (the sum over the kernels it enqueues) from
    committed rocprofv3 counters, or None when absent or taken on other kernel
    sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return int(rec["hbm_bytes_per_launch"])


def calibrate_copy(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--placement", choices=["shuffled", "contiguous"], default=None,
                    help="block placement of the pool for c2, c3 and c5 (default: the "
                         "workload's shuffled free list); contiguous hands out blocks in order, "
                         "to measure what the paged gather costs")
    ap.add_argument("--cold", action="store_true",
                    help="read 512 MB of scratch (more than the 256 MB infinity cache) before "
                         "every step, outside the timing, and time each step alone with HIP "
                         "events: a cache-cold side measurement, not the default line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported and nothing was measured.", flush=True)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return 0

    import paged_kv_cache_14_amd as pa
    if not os.path.exists(pa.library_path()):
        from paged_kv_cache_14_amd.build import build_library
        build_library()
    pa.load_library()
    from workloads import DESCRIPTIONS, make_config

    overrides = {}
    if args.placement is not None:
        if args.workload not in ("c2", "c3", "c5"):
            print("bench.py: --placement applies to c2, c3 and c5", file=sys.stderr)
            return 2
        overrides["placement"] = args.placement
    wl = make_config(args.workload, args.seed, **overrides)
    work = work_figures(wl)
    dev = torch.device("cuda:0")
    tdt = torch.float16 if wl.dtype == "f16" else torch.bfloat16

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q, kp, vp = d16(wl.q), d16(wl.k_pool), d16(wl.v_pool)
    kn, vn, slots = d16(wl.k_new), d16(wl.v_new), d32(wl.slot_mapping)
    bt, cl, qsl = d32(wl.block_tables), d32(wl.context_lens), d32(wl.query_start_loc)
    out = torch.empty_like(q)
    ws_bytes = pa.pa_attention_workspace_size(wl.num_seqs, wl.total_q, wl.num_q_heads,
                                              wl.num_kv_heads, wl.head_dim, wl.max_context_len,
                                              wl.max_query_len)
    ws = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.pa_kv_write(kn, vn, kp, vp, slots, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_attention(q, kp, vp, bt, cl, qsl, wl.num_kv_heads, wl.scale,
                        max_query_len=wl.max_query_len, max_context_len=wl.max_context_len,
                        out=out, workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    scratch = None
    if args.cold:  # read (not written: no dirty lines to write back) before every step
        scratch = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        sink = torch.empty(1, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            torch.sum(scratch, dim=0, keepdim=True, dtype=torch.int64, out=sink)  # evicts the pools
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    kvw_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    attn_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    ms_per_step = wall * 1e3 / args.steps
    if args.cold:  # the wall clock includes the scratch writes: use the steps' own events
        ms_per_step = float(np.mean([a.elapsed_time(c) for a, _, c in evs]))
    step_s = ms_per_step / 1e3
    value = work["kv_bytes"] / step_s / 1e9

    bound = BOUND[args.workload]
    if bound == "hbm":
        achieved = work["kv_bytes"] / (attn_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = work["flops"] / (attn_ms / 1e3) / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["traffic"] = load_traffic(args.workload)
    roof["kernel"] = "pa_attention: " + " + ".join(attention_launches(wl))
    roof["ms_per_launch"] = round(attn_ms, 5)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}"
                        + (f"; {args.placement} placement" if args.placement else "")
                        + ("; infinity cache evicted before every step" if args.cold else ""),
            "seed": wl.meta["seed"],
            "num_seqs": wl.num_seqs,
            "query_tokens": wl.total_q,
            "context_tokens": int(wl.context_lens.sum()),
            "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "num_blocks": wl.num_blocks,
        },
        "query_tokens_per_s": round(work["query_tokens"] / step_s, 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "attention_ms": round(attn_ms, 5),
        "kv_write_ms": round(kvw_ms, 5),
        "attention_tflops": round(work["flops"] / (attn_ms / 1e3) / 1e12, 3),
        "work": work,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del q, kp, vp, kn, vn, out, ws
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
