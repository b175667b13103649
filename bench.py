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

The timed steps are captured into one HIP graph and replayed (as a serving
loop replays its captured decode step), so the device runs them back to back
without waiting for the host; the same steps launched one call at a time are
reported beside them under "eager".
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn KV-read GB/s (% HBM peak) and query tokens/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # dense matrix-core peak
BOUND = {"c1": "hbm", "c2": "hbm", "c3": "hbm", "c4": "hbm", "c5": "mfma"}


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with runs of whitespace folded,
    so that an edit of comments alone keeps the hash (the counters it guards
    depend on the code only)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_14_amd", "csrc", "*"))):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode() + _code_only(f.read()).encode())
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
    decode_only = wl.max_query_len * G <= 8
    if G <= 8:  # sequences with at most 8 rows per KV head may exist
        if decode_only and wl.num_seqs >= 2 and wl.max_context_len > 64:
            names += ["cascade_plan_kernel", "prefill_kernel<shared prefix>"]
        names.append("decode_kernel")
    if not decode_only:
        if not (G <= 8 and wl.num_seqs <= 64):  # else the decode kernel ranks the work
            names.append("prefill_order_kernel")
        # calls with more than 128 query rows per KV head take the wide kernel
        # (its 8-wave form below 1024 rows)
        names.append("prefill_wide_kernel" if wl.max_query_len * G > 128 else "prefill_kernel")
    names.append(f"({int((rows <= 8).sum())} decode / {int((rows > 8).sum())} prefill sequences)")
    return names


def host_description():
    """The host the oracle ran on: CPU model, cores visible, numpy's BLAS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(b.get(k, "")) for k in ("name", "version")).strip() or None
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cores_visible": len(os.sched_getaffinity(0)), "blas": blas}


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
        "host": host_description(),
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
    ap.add_argument("--no-all-configs", dest="all_configs", action="store_false",
                    help="skip the all_configs key (every workload's attention time and "
                         "roofline, GPU only)")
    ap.add_argument("--all-steps", type=int, default=20,
                    help="timed steps per workload in all_configs (other than the headline)")
    ap.add_argument("--swap-layers", type=int, default=0, metavar="L",
                    help="side measurement of the two-tier cache instead of the default line: "
                         "L layers of the workload, part of each layer's K/V in pinned host "
                         "memory, swapped in layer by layer serially and pipelined on a second "
                         "stream")
    ap.add_argument("--swap-fraction", type=float, default=0.0,
                    help="fraction of each layer's blocks swapped in (default: the fraction "
                         "whose transfer takes as long as the layer's attention)")
    ap.add_argument("--quant", action="store_true",
                    help="side measurement instead of the default line: the decode workload "
                         "with every complete 128-token page of cached keys quantized "
                         "(2-bit K and V, promoted key channels at 4 bits), against the same "
                         "decode on 16-bit pages")
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

    if args.quant:
        print(json.dumps(quant_measurement(pa, args.workload, args.steps, args.warmup)),
              flush=True)
        return 0
    if args.swap_layers:
        print(json.dumps(swap_measurement(pa, args.workload, args.swap_layers,
                                          args.swap_fraction, args.steps)), flush=True)
        return 0
    overrides = {}
    if args.placement is not None:
        if args.workload not in ("c2", "c3", "c5"):
            print("bench.py: --placement applies to c2, c3 and c5", file=sys.stderr)
            return 2
        overrides["placement"] = args.placement
    head = measure(pa, args.workload, args.seed, overrides, args.steps, args.warmup, args.cold,
                   keep_workload=not args.no_cpu_baseline)
    wl = head.pop("_workload", None)
    m = head
    step_s = m["ms_per_step"] / 1e3
    value = m["work"]["kv_bytes"] / step_s / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "config": m["config"],
        "query_tokens_per_s": round(m["work"]["query_tokens"] / step_s, 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "attention_ms": m["attention_ms"],
        "kv_write_ms": m["kv_write_ms"],
        "attention_tflops": m["attention_tflops"],
        "timing": m["timing"],
        "eager": m["eager"],
        "work": m["work"],
        "roofline": m["roofline"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    del wl
    if args.all_configs and not args.cold and args.placement is None:
        # Every workload in the same format (attention on the GPU only, no
        # oracle), the headline one included as measured above.
        allc = {}
        for name in ("c1", "c2", "c3", "c4", "c5"):
            if name == args.workload:
                r = m
            else:
                # At least 10 untimed steps: the multi-turn prefill, for one,
                # runs its first steps at a higher clock than the steady state.
                r = measure(pa, name, None, {}, args.all_steps, max(args.warmup, 10), False,
                            keep_workload=False)
            allc[name] = {
                "attention_ms": r["attention_ms"],
                "kv_write_ms": r["kv_write_ms"],
                "ms_per_step": round(r["ms_per_step"], 5),
                "timing": r["timing"],
                "eager": r["eager"],
                "steps": r["steps"],
                "roofline": {k: r["roofline"][k] for k in
                             ("bound", "achieved", "peak", "unit", "frac", "traffic")},
                # both fractions: the prefill workloads sit between the two roofs
                "hbm_frac": round(r["work"]["kv_bytes"] / (r["attention_ms"] / 1e3) / 1e9
                                  / HBM_PEAK_GBS, 4),
                "mfma_frac": round(r["work"]["flops"] / (r["attention_ms"] / 1e3) / 1e12
                                   / MFMA_PEAK_TFLOPS[r["dtype"]], 4),
                "kv_bytes": r["work"]["kv_bytes"],
                "flops": r["work"]["flops"],
                "query_tokens_per_s": round(r["work"]["query_tokens"] / (r["attention_ms"] / 1e3),
                                            1),
                "workload": r["config"]["workload"],
            }
        result["all_configs"] = allc
    print(json.dumps(result), flush=True)
    return 0


def swap_measurement(pa, name, layers, fraction, reps):
    """Two-tier K/V: every layer of `layers` has its own GPU pool; the leading
    blocks of every sequence (a fraction of each layer's blocks, the earliest
    context, which a cost-aware policy evicts first) live in a pinned host
    tier, one contiguous run of blocks per layer, and are swapped in before
    the layer's attention.  Two ways to swap in, timed with HIP events:
      kernel: one pa_swap_blocks launch reads the run across the host link
              and scatters its blocks straight into the pool;
      dma:    pa_swap_in_staged: a copy-engine transfer of the run into a
              device staging buffer, then a scatter from it (device to device).
    Each is run serially (swap-in, then attention, one stream) and pipelined
    (layer i+1's swap-in on a copy stream beside layer i's attention)."""
    import torch
    from workloads import make_config

    wl = checked(pa, make_config(name))
    dev = torch.device("cuda:0")
    tdt = torch.float16 if wl.dtype == "f16" else torch.bfloat16
    Hkv, D = wl.num_kv_heads, wl.head_dim
    block_bytes = 2 * Hkv * 16 * D * 2          # K and V of one block

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    k0, v0 = d16(wl.k_pool), d16(wl.v_pool)
    pa.pa_kv_write(d16(wl.k_new), d16(wl.v_new), k0, v0, d32(wl.slot_mapping))
    q = d16(wl.q)
    bt, cl, qsl = d32(wl.block_tables), d32(wl.context_lens), d32(wl.query_start_loc)
    # Blocks in table order, each sequence's leading ones first.
    order, seen = [], set()
    N = [-(-int(c) // 16) for c in wl.context_lens]
    for j in range(max(N)):
        for s in range(wl.num_seqs):
            if j < N[s]:
                b = int(wl.block_tables[s, j])
                if b not in seen:
                    seen.add(b)
                    order.append(b)
    pools = [(k0.clone(), v0.clone()) for _ in range(layers)]
    out = torch.empty_like(q)
    ws = torch.zeros(max(1, pa.pa_attention_workspace_size(
        wl.num_seqs, wl.total_q, wl.num_q_heads, Hkv, D, wl.max_context_len,
        wl.max_query_len)), dtype=torch.uint8, device=dev)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()

    def attend(i, stream):
        pa.pa_attention(q, pools[i][0], pools[i][1], bt, cl, qsl, Hkv, wl.scale,
                        max_query_len=wl.max_query_len, max_context_len=wl.max_context_len,
                        out=out, workspace=ws, stream=stream)

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(compute)
        for _ in range(n):
            fn()
        b.record(compute)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def host_run(ids):
        """The pinned host run of blocks `ids` of layer 0's pool, in that order."""
        sel = torch.as_tensor(np.array(ids, np.int64), device=dev)
        return (k0.index_select(0, sel).cpu().pin_memory(),
                v0.index_select(0, sel).cpu().pin_memory())

    # Link rates over every unique block of one layer.
    all_ids = d32(np.array(order, np.int32))
    seq_all = d32(np.arange(len(order), dtype=np.int32))
    hk, hv = host_run(order)
    nbytes = len(order) * block_bytes
    kern_full_ms = timed(lambda: pa.pa_swap_blocks(pools[0][0], pools[0][1], hk, hv, seq_all,
                                                   all_ids, stream=compute), 3)
    sk, sv = torch.empty_like(hk, device=dev), torch.empty_like(hv, device=dev)
    dma_full_ms = timed(lambda: (sk.copy_(hk, non_blocking=True),
                                 sv.copy_(hv, non_blocking=True)), 3)
    del hk, hv, sk, sv
    attn_ms = timed(lambda: attend(0, compute), reps)
    if fraction <= 0:
        fraction = min(1.0, attn_ms / dma_full_ms)
    count = max(1, int(round(fraction * len(order))))
    ids = d32(np.array(order[:count], np.int32))
    seq_ids = d32(np.arange(count, dtype=np.int32))
    host = [host_run(order[:count]) for _ in range(layers)]
    staging = [(torch.empty_like(host[0][0], device=dev), torch.empty_like(host[0][1], device=dev))
               for _ in range(layers)]

    def swap_kernel(i, stream):
        pa.pa_swap_blocks(pools[i][0], pools[i][1], host[i][0], host[i][1], seq_ids, ids,
                          stream=stream)

    def swap_dma(i, stream):
        pa.pa_swap_in_staged(pools[i][0], pools[i][1], host[i][0], host[i][1], staging[i][0],
                             staging[i][1], ids, stream=stream)

    landed = [torch.cuda.Event() for _ in range(layers)]

    def serial(swap):
        for i in range(layers):
            swap(i, compute)
            attend(i, compute)

    def pipelined(swap):
        copy.wait_stream(compute)
        for i in range(layers):
            swap(i, copy)
            landed[i].record(copy)
        for i in range(layers):
            compute.wait_event(landed[i])
            attend(i, compute)

    res = {
        "measurement": "two-tier K/V, layer-pipelined swap-in",
        "workload": name,
        "layers": layers,
        "blocks_per_layer": len(order),
        "swapped_blocks_per_layer": count,
        "swap_fraction": round(count / len(order), 4),
        "block_bytes": block_bytes,
        "link_rate_kernel_GBs": round(nbytes / (kern_full_ms / 1e3) / 1e9, 2),
        "link_rate_dma_GBs": round(nbytes / (dma_full_ms / 1e3) / 1e9, 2),
        "attention_ms_per_layer": round(attn_ms, 4),
    }
    for tag, swap in (("kernel", swap_kernel), ("dma", swap_dma)):
        sw = timed(lambda: swap(0, compute), reps)
        se = timed(lambda: serial(swap), max(1, reps // 4))
        pi = timed(lambda: pipelined(swap), max(1, reps // 4))
        res[tag] = {"swap_in_ms_per_layer": round(sw, 4), "serial_ms": round(se, 4),
                    "pipelined_ms": round(pi, 4), "pipelined_vs_serial": round(se / pi, 3),
                    "lower_bound_ms": round(layers * max(sw, attn_ms) + min(sw, attn_ms), 4)}
    # One pipelined run with events on both streams: when each layer's
    # swap-in started and landed (copy stream) and its attention ran (compute
    # stream), in ms from the run's start.
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    base, s_in, s_end, a_in, a_end = ev(), [], [], [], []
    torch.cuda.synchronize()
    base.record(compute)
    copy.wait_stream(compute)
    for i in range(layers):
        s_in.append(ev())
        s_end.append(ev())
        s_in[i].record(copy)
        swap_dma(i, copy)
        s_end[i].record(copy)
    for i in range(layers):
        compute.wait_event(s_end[i])
        a_in.append(ev())
        a_end.append(ev())
        a_in[i].record(compute)
        attend(i, compute)
        a_end[i].record(compute)
    torch.cuda.synchronize()
    res["dma_timeline_ms"] = [
        {"layer": i, "swap_in": [round(base.elapsed_time(s_in[i]), 4),
                                 round(base.elapsed_time(s_end[i]), 4)],
         "attention": [round(base.elapsed_time(a_in[i]), 4),
                       round(base.elapsed_time(a_end[i]), 4)]} for i in range(layers)]
    return res


def quant_measurement(pa, name, steps, warmup):
    """Decode over quantized pages: each sequence's complete 128-token pages of
    cached keys quantized once (timed separately), the rest 16-bit blocks.
    Times pa_attention_quant and pa_attention on the same batch (HIP events);
    the algorithmic bytes of the quantized call are its pages' bytes plus the
    16-bit tail's unique blocks."""
    import torch
    from workloads import make_config

    wl = checked(pa, make_config(name))
    dev = torch.device("cuda:0")
    tdt = torch.float16 if wl.dtype == "f16" else torch.bfloat16
    Hkv, D, B = wl.num_kv_heads, wl.head_dim, wl.block_size
    PT, PB = pa.PA_QPAGE_TOKENS, pa.PA_QPAGE_BYTES

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q, kp, vp = d16(wl.q), d16(wl.k_pool), d16(wl.v_pool)
    pa.pa_kv_write(d16(wl.k_new), d16(wl.v_new), kp, vp, d32(wl.slot_mapping))
    bt, cl, qsl = d32(wl.block_tables), d32(wl.context_lens), d32(wl.query_start_loc)
    n = wl.query_lens
    quant = ((wl.context_lens.astype(np.int64) - n) // PT * PT).astype(np.int32)
    # Pages are per sequence: a block shared by several tables is quantized
    # into each sequence's own page (the shared-prefix path is not used here).
    page_tables = np.full((wl.num_seqs, max(1, int(quant.max()) // PT)), -1, np.int32)
    src, nxt = [], 0
    for s_ in range(wl.num_seqs):
        for p in range(int(quant[s_]) // PT):
            page_tables[s_, p] = nxt
            src.append(wl.block_tables[s_, 8 * p:8 * p + 8])
            nxt += 1
    qpool = torch.zeros((max(1, nxt), Hkv, PB), dtype=torch.uint8, device=dev)
    ids, srcb = d32(np.arange(nxt, dtype=np.int32)), d32(np.array(src, np.int32).reshape(-1, 8))
    out = torch.empty_like(q)
    ws = torch.zeros(max(1, pa.pa_attention_workspace_size(
        wl.num_seqs, wl.total_q, wl.num_q_heads, Hkv, D, wl.max_context_len,
        wl.max_query_len)), dtype=torch.uint8, device=dev)
    pt, ql = d32(page_tables), d32(quant)
    compute = torch.cuda.current_stream()

    def timed(fn, n_):
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(compute)
        for _ in range(n_):
            fn()
        b.record(compute)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n_

    enc_ms = timed(lambda: pa.pa_quantize_pages(qpool, kp, vp, ids, srcb), max(1, steps // 5))
    quant_ms = timed(lambda: pa.pa_attention_quant(
        q, qpool, pt, ql, kp, vp, bt, cl, qsl, Hkv, wl.scale, max_query_len=wl.max_query_len,
        max_context_len=wl.max_context_len, out=out, workspace=ws), steps)
    plain_ms = timed(lambda: pa.pa_attention(
        q, kp, vp, bt, cl, qsl, Hkv, wl.scale, max_query_len=wl.max_query_len,
        max_context_len=wl.max_context_len, out=out, workspace=ws), steps)
    # bytes the quantized call must read: pages + unique 16-bit tail blocks
    tail = set()
    for s_ in range(wl.num_seqs):
        for j in range(int(quant[s_]) // B, -(-int(wl.context_lens[s_]) // B)):
            tail.add(int(wl.block_tables[s_, j]))
    tail_tokens = sum(min(B, int(wl.context_lens[s_]) - j * B)
                      for s_ in range(wl.num_seqs)
                      for j in range(int(quant[s_]) // B, -(-int(wl.context_lens[s_]) // B)))
    q_bytes = nxt * Hkv * PB + len(tail) * Hkv * B * D * 2 * 2
    plain_bytes = work_figures(wl)["kv_bytes"]
    return {
        "measurement": "decode over quantized pages (2-bit K/V, 16 key channels at 4 bits)",
        "workload": name,
        "pages": nxt,
        "quantized_tokens": int(quant.sum()),
        "tail_tokens_16bit": int(tail_tokens),
        "encode_ms": round(enc_ms, 4),
        "encode_us_per_page_head": round(enc_ms * 1e3 / max(1, nxt * Hkv), 4),
        "attention_quant_ms": round(quant_ms, 5),
        "attention_16bit_ms": round(plain_ms, 5),
        "speedup": round(plain_ms / quant_ms, 3),
        "bytes_quant_call": int(q_bytes),
        "bytes_16bit_call": int(plain_bytes),
        "bytes_ratio": round(plain_bytes / q_bytes, 3),
        "quant_call_GBs": round(q_bytes / (quant_ms / 1e3) / 1e9, 2),
        "logical_kv_GBs": round(plain_bytes / (quant_ms / 1e3) / 1e9, 2),
    }


def checked(pa, wl):
    """The workload's tables, lengths, offsets and slots pass the library's
    host check of the kernels' device preconditions before any GPU call."""
    pa.pa_check_batch(wl.block_tables, wl.context_lens, wl.query_start_loc, wl.num_blocks,
                      wl.slot_mapping, slots_are_new_tokens=True)
    return wl


def measure(pa, name, seed, overrides, steps, warmup, cold, keep_workload):
    """Time `steps` kv_write + attention steps of one workload after `warmup`
    untimed ones; HIP events on the stream the kernels run on."""
    import torch
    from workloads import DESCRIPTIONS, make_config

    wl = checked(pa, make_config(name, seed, **overrides))
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

    for _ in range(warmup):
        step()

    # Eager: one call at a time, HIP events between the calls.  For calls of a
    # few microseconds (the single-sequence decode) this includes the
    # binding's per-call host time, which the device waits for.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    scratch = None
    if cold:  # read (not written: no dirty lines to write back) before every step
        scratch = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        sink = torch.empty(1, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            torch.sum(scratch, dim=0, keepdim=True, dtype=torch.int64, out=sink)  # evicts the pools
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager = {"attention_ms": round(float(np.mean([b.elapsed_time(c) for _, b, c in evs])), 5),
             "kv_write_ms": round(float(np.mean([a.elapsed_time(b) for a, b, _ in evs])), 5),
             "ms_per_step": round(wall * 1e3 / steps, 5)}
    if cold:  # the wall clock includes the scratch reads: use the steps' own events
        eager["ms_per_step"] = round(float(np.mean([a.elapsed_time(c) for a, _, c in evs])), 5)

    timing = "eager"
    attn_ms, kvw_ms, ms_per_step = eager["attention_ms"], eager["kv_write_ms"], eager["ms_per_step"]
    if not cold:
        # The timed steps: all `steps` of them captured into one HIP graph
        # (capture is not timed) and replayed once, bracketed by device
        # synchronisation, so that the device runs them back to back as a
        # serving loop replaying its captured step would.  Per-call times of
        # attention and of the K/V write come from graphs of `steps` calls of
        # each (median of three replays, HIP events on the replay stream).
        timing = "hip_graph"
        eager_out = out.clone()

        # (launched on the current stream: inside a capture, the capturing one)
        def attention_only():
            pa.pa_attention(q, kp, vp, bt, cl, qsl, wl.num_kv_heads, wl.scale,
                            max_query_len=wl.max_query_len, max_context_len=wl.max_context_len,
                            out=out, workspace=ws)

        def kv_write_only():
            pa.pa_kv_write(kn, vn, kp, vp, slots)

        def whole_step():
            kv_write_only()
            attention_only()

        def captured(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(steps):
                    fn()
            torch.cuda.synchronize()
            g.replay()  # untimed
            torch.cuda.synchronize()
            return g

        def per_call_ms(fn):
            g = captured(fn)
            times = []
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                b.synchronize()
                times.append(a.elapsed_time(b) / steps)
            del g
            return float(np.median(times))

        g = captured(whole_step)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
        del g
        attn_ms = per_call_ms(attention_only)
        kvw_ms = per_call_ms(kv_write_only)
        torch.cuda.synchronize()
        # the kernels merge in a fixed order: a replay reproduces the eager bits
        if not torch.equal(out.view(torch.int16), eager_out.view(torch.int16)):
            raise RuntimeError(f"{name}: graph replay changed the attention output")
        del eager_out

    bound = BOUND[name]
    if bound == "hbm":
        achieved = work["kv_bytes"] / (attn_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = work["flops"] / (attn_ms / 1e3) / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["traffic"] = load_traffic(name)
    roof["kernel"] = "pa_attention: " + " + ".join(attention_launches(wl))
    roof["ms_per_launch"] = round(attn_ms, 5)
    res = {
        "dtype": wl.dtype,
        "steps": steps,
        "ms_per_step": ms_per_step,
        "attention_ms": round(attn_ms, 5),
        "kv_write_ms": round(kvw_ms, 5),
        "attention_tflops": round(work["flops"] / (attn_ms / 1e3) / 1e12, 3),
        "timing": timing,
        "eager": eager,
        "work": work,
        "roofline": roof,
        "config": {
            "workload": f"{name}: {DESCRIPTIONS[name]}"
                        + (f"; {overrides['placement']} placement" if overrides else "")
                        + ("; infinity cache evicted before every step" if cold else ""),
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
    }
    del q, kp, vp, kn, vn, out, ws, scratch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if keep_workload:
        res["_workload"] = wl
    return res


if __name__ == "__main__":
    sys.exit(main())
