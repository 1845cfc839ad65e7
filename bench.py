#!/usr/bin/env python3
"""Throughput of the ordered fp32 scatter-reduce on one MI355X.

A step is one pass of the hot path over one batch of synthetic input.  For the
default workload, MoE unpermute/combine (T=16384 tokens, 256 experts, top-8,
hidden 7168, bf16 expert outputs), a step is:
  1. dr_sort_by_dest on the routing keys (stable expert-major dispatch order,
     whose inverse permutation is the row of every (token, slot));
  2. dr_combine: gather the 8 rows of every token, fp32 products with the
     gates, the fixed-order sum, one write of the [16384, 7168] fp32 output;
  3. dr_fingerprint of the output (the byte-wise check of a step).
Inputs are resident in HBM before timing starts.  The line printed reports
whole-step throughput in GB/s of algorithmic bytes.  It also reports the
combine kernel against the HBM roofline (timed live with HIP events on the
stream it runs on), the overhead against the atomicAdd baseline, and the CPU
oracle timed on a bounded sample of the same workload.

Other workloads (--workload sparse_attn_dk | embedding_grad | splitk_mhc |
decode_attention | tiny_moe_combine) print the same kind of line for their
own step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ordered scatter-reduce HBM GB/s (% of peak); overhead vs atomicAdd path"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe_combine",
                    choices=["moe_combine", "tiny_moe_combine", "sparse_attn_dk", "embedding_grad", "splitk_mhc",
                             "decode_attention", "sparse_attn_dk_fused", "grouped_wgrad"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone: no comparison legs (atomic, unfused, cold cache, extra entry points) "
                         "and no copy ceiling, so that a profiler's trace holds only the step's kernels")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target duration of the CPU oracle sample")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time the MoE combine only; by default the line also carries a block per other "
                         "configuration (sparse-attention dK index_add and its fused form, embedding-gradient "
                         "index_add, split-K, grouped expert weight gradient)")
    ap.add_argument("--other-cpu-seconds", type=float, default=4.0,
                    help="target duration of each other configuration's CPU oracle sample")
    ap.add_argument("--json-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run a plain fp32 copy kernel of this many MiB (read + write), so that "
                         "profiler byte counters can be scaled against a known transfer")
    return ap.parse_args()


# ---------------------------------------------------------------------------
class Timer:
    """HIP events on the current stream around named phases of each step."""

    def __init__(self, torch, phases):
        self.torch = torch
        self.phases = phases
        self.events = []

    def step(self):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.phases) + 1)]
        self.events.append(evs)
        return evs

    def mean_ms(self):
        self.torch.cuda.synchronize()
        out = {}
        for i, name in enumerate(self.phases):
            out[name] = float(np.mean([e[i].elapsed_time(e[i + 1]) for e in self.events]))
        return out


# ---------------------------------------------------------------------------
def bench_moe(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only=False):
    import oracle
    import workloads
    log(f"{name}: generating inputs")
    inp = workloads.make(name)
    T, E, k, H = inp.T, inp.E, inp.k, inp.H
    elem = 2 if inp.rows_dtype == "bf16" else 4
    keys = torch.from_numpy(inp.expert_ids.reshape(-1).copy()).cuda()
    if inp.rows_dtype == "bf16":
        rows = torch.from_numpy(inp.rows.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        rows = torch.from_numpy(inp.rows).cuda()
    gates = torch.from_numpy(inp.gates).cuda()
    n = T * k
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    seg = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    ws_sort = torch.empty(dr.dr_sort_workspace_size(n, E), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    fp = torch.empty(1, dtype=torch.int64, device="cuda")
    ws_cfp = torch.empty(dr.dr_combine_fingerprinted_workspace_size(rows.dtype, H, T), dtype=torch.uint8,
                         device="cuda")
    row_of = inv.view(T, k)

    combine_bytes = n * H * elem + n * 4 + n * 4 + T * H * 4
    sort_bytes = n * 4 * 3 + (E + 1) * 4
    # algorithmic bytes of the scatter-reduce itself (dispatch sort + combine); the fingerprint
    # check is overhead inside the step's time
    step_bytes = combine_bytes + sort_bytes

    timer = Timer(torch, ["sort", "combine_fingerprinted"])

    def step(evs=None):
        if evs: evs[0].record()
        dr.dr_sort_by_dest(keys, E, perm=perm, seg_offsets=seg, inv_perm=inv, ws=ws_sort)
        if evs: evs[1].record()
        dr.dr_combine_fingerprinted(rows, row_of, gates, out=out, out_hash=fp, ws=ws_cfp)
        if evs: evs[2].record()

    log(f"{name}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    fps = set()
    log(f"{name}: timing {steps} steps")
    t0 = time.perf_counter()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step(timer.step())
    stop.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms_per_step = start.elapsed_time(stop) / steps
    phases = timer.mean_ms()
    fps.add(int(fp.item()))

    # the step's output is the same every replay
    for _ in range(2):
        step()
        fps.add(int(fp.item()))
    assert len(fps) == 1, "combine step output changed between replays"

    # the reported step: captured once in a HIP graph and replayed (the calls launch only kernels on the
    # current stream), so the five launches cost no host time between them
    from bench_workloads import graph_ms
    eager_ms = ms_per_step
    ms_per_step = graph_ms(torch, step, steps, warmup)
    fps.add(int(fp.item()))
    assert len(fps) == 1, "graph replays of the combine step changed its output"

    from bench_workloads import cold_ms, cold_roofline
    extras, extra_roofline = {}, {}
    if not step_only:
        # the same combine without the fused fingerprint, and the separate fingerprint pass
        ws_fp = torch.empty(dr.dr_fingerprint_workspace_size(out.numel() * 4), dtype=torch.uint8, device="cuda")
        ptimer = Timer(torch, ["combine", "fingerprint"])
        for i in range(warmup + steps):
            evs = ptimer.step() if i >= warmup else None
            if evs: evs[0].record()
            dr.dr_combine(rows, row_of, gates, out=out)
            if evs: evs[1].record()
            dr.dr_fingerprint(out, out=fp, ws=ws_fp)
            if evs: evs[2].record()
        plain = ptimer.mean_ms()
        fps.add(int(fp.item()))

        # atomic baseline: zeroing (scatter_add_ needs a zeroed output) + atomic combine
        atimer = Timer(torch, ["zero", "combine_atomic"])
        out_a = torch.empty_like(out)

        def atomic_step(evs=None):
            if evs: evs[0].record()
            out_a.zero_()
            if evs: evs[1].record()
            dr.dr_combine_atomic(rows, row_of, gates, out=out_a)
            if evs: evs[2].record()

        for _ in range(warmup):
            atomic_step()
        for _ in range(steps):
            atomic_step(atimer.step())
        aph = atimer.mean_ms()
        torch.testing.assert_close(out_a, out, rtol=1e-5, atol=1e-5)
        assert len(fps) == 1, "the unfused combine and fingerprint differ from the fused step"

        ms_cold = cold_ms(torch, step)
        comb_cold = cold_ms(torch, lambda: dr.dr_combine_fingerprinted(rows, row_of, gates, out=out, out_hash=fp,
                                                                       ws=ws_cfp))

        # the forward's dispatch-side permute of the same routing: token rows copied to expert-major order
        x = rows[:T]
        out_p = torch.empty(n, H, dtype=rows.dtype, device="cuda")
        for _ in range(warmup):
            dr.dr_permute_rows(x, perm, k, inv_perm=inv, out=out_p)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            dr.dr_permute_rows(x, perm, k, inv_perm=inv, out=out_p)
        e1.record()
        torch.cuda.synchronize()
        perm_ms = e0.elapsed_time(e1) / steps
        perm_bytes = T * H * elem + n * 4 + n * H * elem  # each token row read once at least, every copy written
        del out_p
        extras = {
            "unfused_ms": {k2: round(v, 4) for k2, v in plain.items()},
            "overhead_vs_atomic": {
                "deterministic_combine_ms": round(phases["combine_fingerprinted"], 4),
                "atomic_zero_plus_combine_ms": round(aph["zero"] + aph["combine_atomic"], 4),
                "atomic_combine_only_ms": round(aph["combine_atomic"], 4),
                "overhead": round(phases["combine_fingerprinted"] / (aph["zero"] + aph["combine_atomic"]) - 1, 4),
                "overhead_vs_atomic_kernel_only": round(phases["combine_fingerprinted"] / aph["combine_atomic"] - 1,
                                                        4),
            },
            "cold_cache_ms_per_step": round(ms_cold, 4),
            "dispatch_permute": {"ms": round(perm_ms, 4), "algorithmic_bytes": perm_bytes,
                                 "achieved_gbs": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1)},
        }
        extra_roofline = cold_roofline(combine_bytes, comb_cold)

    comb_ms = phases["combine_fingerprinted"]
    achieved = combine_bytes / (comb_ms * 1e-3) / 1e9
    from bench_workloads import measured_traffic, source_digest
    digest = source_digest("combine.hip", "device.h")
    result = {
        "ms_per_step": ms_per_step,
        "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "config": {"workload": f"{name}: MoE unpermute/combine T={T} tokens, {E} experts, top-{k}, hidden {H}, "
                               f"{inp.rows_dtype} expert outputs, fp32 out",
                   "tokens": T, "experts": E, "top_k": k, "hidden": H,
                   "step": "dispatch sort + ordered combine with the output fingerprint taken as it is stored",
                   "step_algorithmic_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "combine_kernel (fingerprinting) + its 1-workgroup final sum",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("combine_kernel_fp", name, digest),
                     "algorithmic_bytes_per_launch": combine_bytes, "avg_launch_ms": round(comb_ms, 4),
                     **extra_roofline},
        "phases_ms": {k2: round(v, 4) for k2, v in phases.items()},
        "timing": "step replayed from a HIP graph; eager_ms_per_step with HIP events between the calls",
        "eager_ms_per_step": round(eager_ms, 4),
        "eager_wall_ms_per_step": round(wall_ms, 4),
        **extras,
    }
    if want_cpu:
        result["cpu_baseline"] = cpu_baseline_moe(oracle, inp, cpu_seconds)
    return result


def cpu_baseline_moe(oracle, inp, seconds):
    """The oracle (C) timed on a bounded sample of tokens, on one thread and on the host's cores (token
    ranges per thread; the bits must not change)."""
    from bench_workloads import host_threads
    _, _, inv = oracle.sort_by_dest(inp.expert_ids.reshape(-1), inp.E)
    row_of = inv.reshape(inp.T, inp.k)
    elem = 2 if inp.rows_dtype == "bf16" else 4
    per_token = inp.k * inp.H * elem + inp.k * 8 + inp.H * 4
    probe = np.arange(min(16, inp.T))
    t0 = time.perf_counter()
    oracle.combine(inp.rows, row_of, inp.gates, tokens=probe)
    dt = max(time.perf_counter() - t0, 1e-6) / len(probe)
    count = int(min(inp.T, max(len(probe), seconds / dt)))
    tokens = np.arange(count)
    log(f"cpu baseline: oracle combine on {count} tokens (~{count * dt:.1f} s)")
    t0 = time.perf_counter()
    one = oracle.combine(inp.rows, row_of, inp.gates, tokens=tokens)
    el = time.perf_counter() - t0
    th = host_threads()
    t0 = time.perf_counter()
    many = oracle.combine(inp.rows, row_of, inp.gates, tokens=tokens, threads=th)
    el_mt = time.perf_counter() - t0
    same = bool(np.array_equal(one.view(np.uint32), many.view(np.uint32)))
    if not same:
        raise RuntimeError("the oracle's bits changed with its thread count")
    return {"value": round(per_token * count / el_mt / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
            "sample": f"first {count} of {inp.T} tokens of the same workload (combine only); {th} threads "
                      f"{el_mt:.1f} s, 1 thread {el:.1f} s",
            "seconds": round(el_mt, 2),
            "single_thread": {"value": round(per_token * count / el / 1e9, 4), "cores": 1, "seconds": round(el, 2)},
            "bits_identical_across_thread_counts": same}


# ---------------------------------------------------------------------------
def copy_ceiling(torch, achieved_gbs: float, mib: int = 2048, reps: int = 5) -> dict:
    """A 2 GiB device-to-device copy by an elementwise kernel (read + write),
    timed with events: the practical HBM ceiling of a plain stream on this
    device, reported next to the datasheet peak.  (torch's copy_ of equal
    dtypes goes to the runtime's blit kernel, which is slower.)"""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        e0.record()
        torch.mul(a, 1.0, out=b)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    ms = sorted(ts)[len(ts) // 2]
    gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    return {"copy_ceiling_gbs": round(gbs, 1), "frac_of_copy": round(achieved_gbs / gbs, 4)}


def host_description() -> dict:
    """The host the CPU baseline ran on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpu": model, "host_logical_cpus": os.cpu_count()}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import bitwise_deterministic_fp32_amd as dr
    torch.cuda.set_device(0)
    dr.dr_set_launch_params(reset=True)
    name = args.workload
    if name in ("moe_combine", "tiny_moe_combine"):
        res = bench_moe(torch, dr, name, args.steps, args.warmup, args.cpu_seconds, not args.no_cpu_baseline,
                        args.step_only)
    else:
        import bench_workloads
        res = bench_workloads.run(torch, dr, name, args.steps, args.warmup, args.cpu_seconds,
                                  not args.no_cpu_baseline, args.step_only)
    if not args.step_only and res["roofline"]["unit"] == "GB/s":
        res["roofline"].update(copy_ceiling(torch, res["roofline"]["achieved"]))
    others = {}
    if name == "moe_combine" and not args.step_only and not args.no_other_configs:
        import bench_workloads
        for other in ("sparse_attn_dk", "embedding_grad", "splitk_mhc", "grouped_wgrad"):
            r = bench_workloads.run(torch, dr, other, args.steps, args.warmup, args.other_cpu_seconds,
                                    not args.no_cpu_baseline, False)
            if "cpu_baseline" in r:
                r["cpu_baseline"].update(host_description())
            r["value_gbs" if r["roofline"]["unit"] == "GB/s" else "value"] = round(r.pop("value"), 2)
            r["ms_per_step"] = round(r["ms_per_step"], 4)
            others[other] = r
            torch.cuda.empty_cache()
    if "cpu_baseline" in res:
        res["cpu_baseline"].update(host_description())
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(2):
            torch.mul(a, 1.0, out=b)  # elementwise copy: reads and writes n*4 bytes
        torch.cuda.synchronize()
        del a, b
    line = {"metric": METRIC, "value": round(res.pop("value"), 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res.pop("ms_per_step"), 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded numpy PCG64 draws of the configuration's shapes and distributions)"}
    line.update(res)
    if others:
        line["other_configs"] = others
    text = json.dumps(line)
    print(text, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
