"""Benchmark of the paged-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one paged GQA decode pass (split + combine) over the bf16 workload
B=64, Hq=32, Hk=8, D=128, seq_lens ~ U{1024..4096}, 64-row blocks behind a
shuffled block_table.  `value` is the KV bytes the step must read (valid K and
V rows) divided by the measured time per step.  Inputs are resident in HBM
before the timed region; consecutive steps read different copies of the KV
pool, so no step is served from the 256 MB last-level cache by its
predecessor.  The other workloads (fp8 KV decode, MLA prefill, block-sparse
prefill, fp8 MLA prefill with per-tensor and blockwise scales, MLA prefill
with an fp8 rope key, chunked
prefill over a bf16 and over an fp8 e4m3fn cache, and a long-context chunk
whose few query tiles are split along the keys) are measured the same way
and reported under "secondary".

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix cores, TFLOP/s
METRIC = "paged decode KV-read GB/s (% HBM peak); MLA prefill TFLOP/s (% MFMA peak)"
ROT_BYTES = 768 << 20          # keep the rotating copies larger than the last-level cache


# Sources whose text decides each measured kernel's code (a change makes the
# stored hardware-counter traffic for that kernel stale).
KERNEL_SOURCES = {
    "decode": ("dev.hpp", "status.hpp", "decode.hip"),
    "prefill": ("dev.hpp", "status.hpp", "prefill.hip"),
}


def _strip_comments(src: str) -> str:
    """C/C++ source without comments and with runs of whitespace collapsed,
    so that a change to the prose of a file does not make its counters stale
    (string literals holding comment markers do not occur in these files)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def _kernel_source_hash(kind: str = "decode") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        p = os.path.join(ROOT, "gqa_attention_paged_amd", "csrc", f)
        if os.path.exists(p):
            with open(p, encoding="utf-8") as fh:
                h.update(_strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def _kind_of(workload: str) -> str:
    """Source set of the workload's dominant kernel: short chunks (plain and
    MLA) run on the decode workers, the rest on the prefill kernel."""
    return "prefill" if workload.startswith("prefill") else "decode"


def _traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary (profiles/traffic.json), or None when it is
    missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as fh:
            t = json.load(fh)
        ent = t.get("workloads", {}).get(workload)
        if not ent or ent.get("source_hash") != _kernel_source_hash(_kind_of(workload)):
            return None
        return ent["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


# Dominant kernel of each workload, as rocprofv3 names it (substring match).
DOMINANT_KERNEL = {
    "decode_gqa_bf16": "decode_worker_mfma<128, false, false>",
    "decode_long_fp8": "decode_worker_mfma<128, true, false>",
    "decode_tiny_fp32": "decode_worker_f32",
    "prefill_mla_bf16": "prefill_fwd<64, false, 0>",
    "prefill_blocksparse_bf16": "prefill_fwd<0, false, 0>",
    "prefill_chunk_bf16": "prefill_fwd<0, true, 0>",
    "prefill_chunk_mla_bf16": "prefill_fwd<64, true, 0>",
    "prefill_mla_fp8": "prefill_fwd<64, false, 1>",
    "prefill_mla_fp8_blockwise": "prefill_fwd<64, false, 2>",
    "prefill_chunk_long_mla_bf16": "prefill_fwd<64, true, 0>",
    "prefill_chunk_fp8kv": "prefill_fwd<0, true, 3>",
    "prefill_mla_rope_fp8": "prefill_fwd<64, false, 4>",
    "decode_mt1_bf16": "decode_worker_mfma<128, false, true>",
    "decode_mt2_bf16": "decode_worker_mfma<128, false, true>",
    "decode_mt4_bf16": "decode_worker_mfma<128, false, true>",
    "decode_mt2_mla_bf16": "decode_worker_rope<false>",
}


def prefill_peak_tflops(case) -> float:
    """The matrix-core peak for the prefill's mix of products: with fp8 inputs
    the nope part of Q.K (Dn of the Dqk + Dv multiply-adds per visible pair
    and head) runs at the fp8 rate and the rope part and P.V at the bf16 rate,
    so the peak is the harmonic mix of the two; bf16 cases get the bf16 peak."""
    if getattr(case, "dtype", "bf16") != "e4m3fn":
        return BF16_MFMA_PEAK_TFLOPS
    f8 = case.D_nope / (case.D_qk + case.D_v)
    return 1.0 / (f8 / FP8_MFMA_PEAK_TFLOPS + (1.0 - f8) / BF16_MFMA_PEAK_TFLOPS)
COPY_KERNEL = "neg_kernel"   # torch.neg(out=) over float32: reads and writes each byte once


def _counter_per_dispatch(csv_dir: str, counter: str):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter CSV."""
    import csv
    import glob
    per = {}
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {csv_dir}")
    for fn in files:
        with open(fn) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def _mean_for(per, pattern: str) -> float:
    vals = [v for name, vs in per.items() if pattern in name for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r}; kernels seen: {sorted(per)[:8]}")
    return sum(vals) / len(vals)


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int, out_path: str) -> dict:
    """Turn a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch) into HBM
    bytes per launch of the workload's dominant kernel, each counter scaled
    by what it reads for the plain copy kernel of `copy_bytes` bytes."""
    from workloads import gen
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    f_copy, w_copy = _mean_for(fetch, COPY_KERNEL), _mean_for(write, COPY_KERNEL)
    k_fetch = copy_bytes / (f_copy * 1024.0)
    k_write = copy_bytes / (w_copy * 1024.0)
    kern = DOMINANT_KERNEL[workload]
    f_k, w_k = _mean_for(fetch, kern), _mean_for(write, kern)
    case = gen.CONFIGS[workload]()
    alg = (case.kv_bytes() if hasattr(case, "kv_bytes") else
           gen.kv_read_bytes(case) if workload.startswith("decode_mt") else None)
    ent = {
        "kernel": kern, "source_hash": _kernel_source_hash(_kind_of(workload)),
        "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k,
        "copy_bytes": copy_bytes, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": k_fetch, "write_scale": k_write,
        "hbm_bytes_per_launch": f_k * 1024.0 * k_fetch + w_k * 1024.0 * k_write,
        "algorithmic_bytes_per_launch": alg,
    }
    t = {"workloads": {}}
    if os.path.exists(out_path):
        with open(out_path) as fh:
            t = json.load(fh)
    t.setdefault("workloads", {})[workload] = ent
    with open(out_path, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return ent


def stats_summary(stats_csv: str, command: str) -> str:
    """A short text table of a rocprofv3 --stats kernel summary."""
    import csv
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    lines = [f"command: {command}", "", f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                     f"{float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.2f}  {r['Name'][:110]}")
    return "\n".join(lines) + "\n"


def _timed_loop(run, steps: int, warmup: int, torch):
    """Warm up, then time exactly `steps` calls with nothing else in the loop
    (wall clock, synchronised on both sides).  A second pass of the same
    `steps` calls brackets each call with HIP events on the current stream
    (the stream the library launches on) for the per-call duration and its
    spread; those events stay out of the first, timed pass."""
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        run(i)
        ends[i].record()
    torch.cuda.synchronize()
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return (t1 - t0) * 1e3 / steps, sum(ev_ms) / len(ev_ms), sorted(ev_ms)


def bench_decode(case, steps, warmup, torch, gq, gu, check=True, warm=False):
    dd = gu.DeviceDecode(case)
    pool_bytes = 2 * dd.k.numel() * dd.k.element_size()
    nrot = max(2, math.ceil(ROT_BYTES / max(1, pool_bytes)) + 1)
    pools = [(dd.k, dd.v)] + [(dd.k.clone(), dd.v.clone()) for _ in range(nrot - 1)]
    plan = dd.plan

    def run(i):
        k, v = pools[i % nrot]
        gq.gqap_paged_decode(plan, dd.q, k, v, dd.bt, dd.sl, case.scale, case.k_scale, case.v_scale, dd.out,
                             dd.lse, dd.ws, plan.workspace_bytes)

    ms_step, ms_ev, evs = _timed_loop(run, steps, warmup, torch)
    # Warm (--warm only): the same pool on every call, so what the 256 MB
    # last-level cache kept of the previous call serves part of the next;
    # reported beside the cold figure, never as it, and left out of the
    # default run so that a kernel trace of it times cold calls only.
    ms_warm = _timed_loop(lambda i: run(0), steps, warmup, torch)[1] if warm else None
    err = None
    if check:
        from oracle import attention as O
        out, _ = dd.results()
        sample = list(range(0, case.B, max(1, case.B // 4)))[:4]
        ref, _ = O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.scale,
                                q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                v_scale=case.v_scale, batches=sample)
        err = float(abs(out[sample] - ref).max())
    nbytes = case.kv_bytes()
    return {
        "workload": case.name, "bytes": nbytes, "ms_per_step": ms_step, "ms_kernel": ms_ev,
        "ms_kernel_p10": evs[len(evs) // 10], "ms_kernel_p90": evs[(9 * len(evs)) // 10],
        "gbs_step": nbytes / (ms_step * 1e-3) / 1e9, "gbs_kernel": nbytes / (ms_ev * 1e-3) / 1e9,
        "workers": plan.num_workers, "rotating_copies": nrot,
        "ms_kernel_warm": ms_warm, "gbs_kernel_warm": nbytes / (ms_warm * 1e-3) / 1e9 if warm else None,
        "max_abs_err_sample": err,
    }


def bench_prefill(case, steps, warmup, torch, gq, gu, check=True):
    dp = gu.DevicePrefill(case)

    def run(i):
        dp.run()

    ms_step, ms_ev, evs = _timed_loop(run, steps, warmup, torch)
    err = None
    if check:
        from oracle import attention as O
        import numpy as np
        out, _ = dp.results()
        rows = np.linspace(0, case.T - 1, 48).astype(np.int64)
        if getattr(case, "rope_dtype", "bf16") == "e4m3fn":
            ref, _ = O.ragged_prefill_rope_fp8(case.q, case.k, case.v, case.k_rope, case.k_rope_scale,
                                               case.cu_seqlens, case.scale, block_mask=case.block_mask, rows=rows)
        elif case.dtype == "e4m3fn":
            ref, _ = O.ragged_prefill_fp8(case.q, case.q_rope, case.k, case.v, case.k_rope, case.cu_seqlens,
                                          case.scale, case.q_scale, case.k_scale, block_mask=case.block_mask,
                                          rows=rows)
        else:
            ref, _ = O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, k_rope=case.k_rope,
                                      block_mask=case.block_mask, dtype="bf16", rows=rows)
        err = float(abs(out[rows] - ref).max())
    flops = case.flops()
    return {
        "workload": case.name, "flops": flops, "ms_per_step": ms_step, "ms_kernel": ms_ev,
        "ms_kernel_p10": evs[len(evs) // 10], "ms_kernel_p90": evs[(9 * len(evs)) // 10],
        "tflops_step": flops / (ms_step * 1e-3) / 1e12, "tflops_kernel": flops / (ms_ev * 1e-3) / 1e12,
        "max_abs_err_sample": err,
    }


def bench_chunk(case, steps, warmup, torch, gq, gu, check=True):
    """A step of chunked prefill: append the chunk into the paged cache, then
    attend (both launches; the append rewrites the same rows every step)."""
    dc = gu.DeviceChunk(case)

    def run(i):
        dc.append()
        dc.run()

    ms_step, ms_ev, evs = _timed_loop(run, steps, warmup, torch)
    err = None
    if check:
        from oracle import attention as O
        import numpy as np
        out, _ = dc.results()
        fp8 = dict(kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
        pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table,
                            case.cu_seqlens_q, case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool, **fp8)
        rows = np.linspace(0, case.T - 1, 48).astype(np.int64)
        ref, _ = O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q, case.kv_lens,
                                 case.scale, dtype="bf16", rows=rows, kr_pool=pools[2] if len(pools) == 3 else None,
                                 **fp8)
        err = float(abs(out[rows] - ref).max())
    flops = case.flops()
    return {
        "workload": case.name, "flops": flops, "ms_per_step": ms_step, "ms_kernel": ms_ev,
        "ms_kernel_p10": evs[len(evs) // 10], "ms_kernel_p90": evs[(9 * len(evs)) // 10],
        "tflops_step": flops / (ms_step * 1e-3) / 1e12, "tflops_kernel": flops / (ms_ev * 1e-3) / 1e12,
        "max_abs_err_sample": err,
    }


def bench_mtdecode(case, steps, warmup, torch, gq, gu, check=True):
    """Multi-token decode: the chunk's new tokens are already in the paged
    cache (appended once, outside the timing); a step is the attention call.
    Reported as cache bytes read per second (every key's K and V of every KV
    head, plus the shared rope row), against the HBM peak."""
    from workloads import gen
    dc = gu.DeviceChunk(case)
    dc.append()

    def run(i):
        dc.run()

    ms_step, ms_ev, evs = _timed_loop(run, steps, warmup, torch)
    err = None
    if check:
        from oracle import attention as O
        out, _ = dc.results()
        pools = dc.pools_bits()
        rows = list(range(0, case.T, max(1, case.T // 48)))
        ref, _ = O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q, case.kv_lens,
                                 case.scale, dtype="bf16", rows=rows, kr_pool=pools[2] if len(pools) == 3 else None)
        err = float(abs(out[rows] - ref).max())
    nbytes = gen.kv_read_bytes(case)
    return {
        "workload": case.name, "bytes": nbytes, "q_len": int(case.q_lens.max()), "ms_per_step": ms_step,
        "ms_kernel": ms_ev, "ms_kernel_p10": evs[len(evs) // 10], "ms_kernel_p90": evs[(9 * len(evs)) // 10],
        "gbs_step": nbytes / (ms_step * 1e-3) / 1e9, "gbs_kernel": nbytes / (ms_ev * 1e-3) / 1e9,
        "splits": int(dc.plan.num_splits), "kernel": DOMINANT_KERNEL.get(case.name), "plan_kernel": int(dc.plan.kernel),
        "max_abs_err_sample": err,
    }


def cpu_baseline_decode(case, budget_s: float = 12.0):
    """The oracle, as it is, on the host: whole decode passes over the same
    workload until about `budget_s` seconds have run (at least one)."""
    ncores = len(os.sched_getaffinity(0))
    from oracle import attention as O
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.scale,
                       q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": case.kv_bytes() * reps / dt / 1e9, "unit": "GB/s", "cores": ncores, "kind": "oracle",
            "sample": f"{reps} full fp64 decode pass(es) over the same {case.B}-sequence workload, {dt:.1f} s"}


def cpu_baseline_full(case):
    """One full evaluation of the oracle, as it is, on the host for a secondary
    workload: every sequence (decode) or every row (prefill, chunked prefill:
    the append and the attention), cut into pieces that run in worker threads
    with one BLAS thread each.  Reported in the workload's own unit, from the
    same numerator as the GPU figure."""
    from oracle import attention as O
    from oracle import parallel as OP
    from workloads import gen
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    if isinstance(case, gen.DecodeCase):
        OP.all_batches(lambda bb: O.paged_decode(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                                                 case.scale, q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                                                 k_scale=case.k_scale, v_scale=case.v_scale, batches=bb),
                       case.B, workers=workers)
        dt = time.perf_counter() - t0
        return {"value": case.kv_bytes() / dt / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
                "sample": f"one full fp64 decode of all {case.B} sequences, {dt:.1f} s"}
    if isinstance(case, gen.ChunkCase):
        fp8 = dict(kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)
        pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table,
                            case.cu_seqlens_q, case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool, **fp8)
        OP.all_rows(lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q,
                                               case.kv_lens, case.scale, dtype="bf16", rows=rr,
                                               kr_pool=pools[2] if len(pools) == 3 else None, **fp8),
                    case.T, block=64, workers=workers)
        what = f"one full fp64 append and chunked prefill of all {case.T} query rows"
    elif getattr(case, "rope_dtype", "bf16") == "e4m3fn":
        OP.all_rows(lambda rr: O.ragged_prefill_rope_fp8(case.q, case.k, case.v, case.k_rope, case.k_rope_scale,
                                                         case.cu_seqlens, case.scale, block_mask=case.block_mask,
                                                         rows=rr), case.T, workers=workers)
        what = f"one full fp64 prefill of all {case.T} rows"
    elif case.dtype == "e4m3fn":
        OP.all_rows(lambda rr: O.ragged_prefill_fp8(case.q, case.q_rope, case.k, case.v, case.k_rope,
                                                    case.cu_seqlens, case.scale, case.q_scale, case.k_scale,
                                                    block_mask=case.block_mask, rows=rr), case.T, workers=workers)
        what = f"one full fp64 prefill of all {case.T} rows"
    else:
        OP.all_rows(lambda rr: O.ragged_prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale,
                                                k_rope=case.k_rope, block_mask=case.block_mask, dtype="bf16",
                                                rows=rr), case.T, workers=workers)
        what = f"one full fp64 prefill of all {case.T} rows"
    dt = time.perf_counter() - t0
    return {"value": case.flops() / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{what}, {dt:.1f} s"}


def cpu_baseline_mtdecode(case):
    """One full oracle evaluation of a multi-token decode workload (the
    append and the attention of every query row), in the workload's unit."""
    from oracle import attention as O
    from oracle import parallel as OP
    from workloads import gen
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    pools = O.append_kv(case.k_new, case.v_new, case.k_pool, case.v_pool, case.block_table, case.cu_seqlens_q,
                        case.kv_lens, kr_new=case.kr_new, kr_pool=case.kr_pool)
    OP.all_rows(lambda rr: O.chunk_prefill(case.q, pools[0], pools[1], case.block_table, case.cu_seqlens_q,
                                           case.kv_lens, case.scale, dtype="bf16", rows=rr,
                                           kr_pool=pools[2] if len(pools) == 3 else None),
                case.T, block=max(1, case.T // workers), workers=workers)
    dt = time.perf_counter() - t0
    return {"value": gen.kv_read_bytes(case) / dt / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"one full fp64 append and attention of all {case.T} query rows, {dt:.1f} s"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="also time the decodes on one pool (last-level cache warm), beside the cold figure")
    ap.add_argument("--only-primary", action="store_true", help="measure only the primary decode workload")
    ap.add_argument("--only", default=None,
                    help="measure one workload by name (for profiling) and print its record instead")
    ap.add_argument("--copy-calibration-bytes", type=int, default=0,
                    help="after the workload, run a plain float32 copy kernel (torch.neg) over this many bytes "
                         "three times: the known-size reference for hardware byte counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="summarise a FETCH_SIZE run and a WRITE_SIZE run of `--only WORKLOAD "
                         "--copy-calibration-bytes N` into profiles/traffic.json (no GPU needed)")
    ap.add_argument("--stats-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "COMMAND"), default=None,
                    help="print a rocprofv3 --stats kernel summary as a short text table (no GPU needed)")
    args = ap.parse_args(argv)
    if args.pmc_summary:
        ent = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.only, args.copy_calibration_bytes,
                          os.path.join(ROOT, "profiles", "traffic.json"))
        print(json.dumps(ent, indent=1))
        return 0
    if args.stats_summary:
        print(stats_summary(*args.stats_summary), end="")
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this library has no "
              "multi-GPU path: each GPU would run the same kernels on its own share).", file=sys.stderr)
        return 2

    import torch
    import gqa_attention_paged_amd as gq
    from workloads import device as gu
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    if args.only:
        mk = gen.CONFIGS[args.only]
        c = mk()
        fn = (bench_prefill if isinstance(c, gen.PrefillCase) else
              bench_mtdecode if args.only.startswith("decode_mt") else
              bench_chunk if isinstance(c, gen.ChunkCase) else bench_decode)
        print(json.dumps(fn(c, args.steps, args.warmup, torch, gq, gu)), flush=True)
        if args.copy_calibration_bytes:
            n = args.copy_calibration_bytes // 4
            src = torch.ones(n, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
        return 0

    case = gen.decode_gqa_bf16()
    prim = bench_decode(case, args.steps, args.warmup, torch, gq, gu, warm=args.warm)
    secondary = [dict(prim, role="primary")]
    if not args.only_primary:
        c4 = gen.decode_long_fp8()
        r4 = bench_decode(c4, args.steps, args.warmup, torch, gq, gu, warm=args.warm)
        r4["roofline"] = {"bound": "hbm", "achieved": r4["gbs_kernel"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": r4["gbs_kernel"] / HBM_PEAK_GBS,
                          "traffic": _traffic("decode_long_fp8")}
        r4["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_full(c4)
        secondary.append(r4)
        del c4
        if hasattr(gu, "DevicePrefill"):
            for mk in (gen.prefill_mla_bf16, gen.prefill_blocksparse_bf16, gen.prefill_mla_fp8,
                       gen.prefill_mla_fp8_blockwise, gen.prefill_mla_rope_fp8):
                pc = mk()
                rp = bench_prefill(pc, args.steps, args.warmup, torch, gq, gu)
                peak = prefill_peak_tflops(pc)
                rp["roofline"] = {"bound": "mfma", "achieved": rp["tflops_kernel"], "peak": round(peak, 1),
                                  "unit": "TFLOP/s", "frac": rp["tflops_kernel"] / peak,
                                  "traffic": _traffic(pc.name)}
                rp["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_full(pc)
                secondary.append(rp)
                del pc
        if hasattr(gu, "DeviceChunk"):
            # the fp8-cache chunk widens its codes to bf16 before the matrix
            # cores, so every chunk workload is priced at the bf16 peak
            for mk in (gen.prefill_chunk_bf16, gen.prefill_chunk_mla_bf16, gen.prefill_chunk_long_mla_bf16,
                       gen.prefill_chunk_fp8kv):
                cc = mk()
                rc = bench_chunk(cc, args.steps, args.warmup, torch, gq, gu)
                rc["roofline"] = {"bound": "mfma", "achieved": rc["tflops_kernel"], "peak": BF16_MFMA_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": rc["tflops_kernel"] / BF16_MFMA_PEAK_TFLOPS,
                                  "traffic": _traffic(cc.name)}
                rc["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_full(cc)
                secondary.append(rc)
                del cc
            # multi-token decode over the paged-decode workload's cache shape (and its MLA form)
            for wl in ("decode_mt1_bf16", "decode_mt2_bf16", "decode_mt4_bf16", "decode_mt2_mla_bf16"):
                mc = gen.CONFIGS[wl]()
                rm = bench_mtdecode(mc, args.steps, args.warmup, torch, gq, gu)
                rm["roofline"] = {"bound": "hbm", "achieved": rm["gbs_kernel"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": rm["gbs_kernel"] / HBM_PEAK_GBS, "traffic": _traffic(mc.name)}
                rm["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_mtdecode(mc)
                secondary.append(rm)
                del mc

    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(case)
    line = {
        "metric": METRIC,
        "value": round(prim["gbs_step"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "paged GQA decode, bf16: B=64, Hq=32, Hk=8, D=128, one query token per sequence, "
                        "seq_lens ~ U{1024..4096}, 64-row blocks, shuffled block_table",
            "kv_bytes_per_step": prim["bytes"],
            "workers": prim["workers"],
            "device": props.name,
            "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(prim["gbs_kernel"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(prim["gbs_kernel"] / HBM_PEAK_GBS, 4),
            "traffic": _traffic("decode_gqa_bf16"),
        },
        "cpu_baseline": cpu,
        "secondary": secondary,
        "kernel_source_hash": {k: _kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
