"""Benchmark of the paged-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one paged GQA decode pass (split + combine) over the bf16 workload
B=64, Hq=32, Hk=8, D=128, seq_lens ~ U{1024..4096}, 64-row blocks behind a
shuffled block_table.  `value` is the KV bytes the step must read (valid K and
V rows) divided by the measured time per step.  Inputs are resident in HBM
before the timed region; consecutive steps read different copies of the KV
pool, so no step is served from the 256 MB last-level cache by its
predecessor.  The other workloads (fp8 KV decode, MLA prefill, block-sparse
prefill) are measured the same way and reported under "secondary".

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
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
METRIC = "paged decode KV-read GB/s (% HBM peak); MLA prefill TFLOP/s (% MFMA peak)"
ROT_BYTES = 768 << 20          # keep the rotating copies larger than the last-level cache


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("dev.hpp", "decode.hip", "prefill.hip"):
        p = os.path.join(ROOT, "gqa_attention_paged_amd", "csrc", f)
        if os.path.exists(p):
            with open(p, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, per_launch_units: float):
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        with open(p) as fh:
            t = json.load(fh)
        ent = t.get(kernel)
        if not ent or ent.get("source_hash") != _kernel_source_hash():
            return None
        return ent["hbm_bytes_per_launch"]
    except Exception:
        return None


def _timed_loop(run, steps: int, warmup: int, torch):
    """Warm up, then time exactly `steps` calls; per-call HIP events on the
    current stream give the kernel-side duration."""
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        run(i)
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return (t1 - t0) * 1e3 / steps, sum(ev_ms) / len(ev_ms), sorted(ev_ms)


def bench_decode(case, steps, warmup, torch, gq, gu, check=True):
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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true", help="measure only the primary decode workload")
    ap.add_argument("--only", default=None,
                    help="measure one workload by name (for profiling) and print its record instead")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this library has no "
              "multi-GPU path: each GPU would run the same kernels on its own share).", file=sys.stderr)
        return 2

    import torch
    import gqa_attention_paged_amd as gq
    from tests import gpu_util as gu
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    if args.only:
        mk = gen.CONFIGS[args.only]
        c = mk()
        fn = bench_prefill if isinstance(c, gen.PrefillCase) else bench_decode
        print(json.dumps(fn(c, args.steps, args.warmup, torch, gq, gu)), flush=True)
        return 0

    case = gen.decode_gqa_bf16()
    prim = bench_decode(case, args.steps, args.warmup, torch, gq, gu)
    secondary = [dict(prim, role="primary")]
    if not args.only_primary:
        c4 = gen.decode_long_fp8()
        r4 = bench_decode(c4, args.steps, args.warmup, torch, gq, gu)
        r4["roofline"] = {"bound": "hbm", "achieved": r4["gbs_kernel"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": r4["gbs_kernel"] / HBM_PEAK_GBS,
                          "traffic": _traffic("decode_long_fp8", 1)}
        secondary.append(r4)
        del c4
        if hasattr(gu, "DevicePrefill"):
            for mk in (gen.prefill_mla_bf16, gen.prefill_blocksparse_bf16):
                pc = mk()
                rp = bench_prefill(pc, args.steps, args.warmup, torch, gq, gu)
                rp["roofline"] = {"bound": "mfma", "achieved": rp["tflops_kernel"], "peak": BF16_MFMA_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": rp["tflops_kernel"] / BF16_MFMA_PEAK_TFLOPS,
                                  "traffic": None}
                secondary.append(rp)
                del pc

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
            "traffic": _traffic("decode_gqa_bf16", 1),
        },
        "cpu_baseline": cpu,
        "secondary": secondary,
        "kernel_source_hash": _kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
