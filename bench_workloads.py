"""bench.py's steps for the index_add and split-K configurations.

sparse_attn_dk / embedding_grad: a step is dr_index_add_fingerprinted (stable
  sort of the contributions by destination, tile plan, ordered segmented
  reduction, destination update), which also moves the destination's
  fingerprint by the change of the rows it rewrites.  The destination keeps
  accumulating from step to step; resetting it is not part of the method.  The
  same step with dr_index_add and a full dr_fingerprint of the destination, and
  the reused-plan time (sort done once, as when the indices are known a step
  early), are reported beside it.
grouped_wgrad: a step is dr_grouped_wgrad (plan, tile kernel, chunk merge): the
  weight gradient of 8 experts (the hottest of the MoE routing, one GPU's share
  at expert parallelism 32: 86,165 token rows), M = 7168, N = 2048, private
  slots of 2048 tokens merged in slot order.  MFMA-bound: reported in TFLOP/s
  against the bf16 dense peak.
splitk_mhc: a step is dr_splitk_gemm_tn (64 private fp32 partials by bf16
  MFMA) and dr_splitk_reduce_fingerprinted (the reduce in split-id order,
  hashing dW as it stores it).
decode_attention: a step is dr_decode_attention (chunk partials over the
  head-major KV cache with a fixed 512-token partition, then the merge in
  chunk order) and dr_fingerprint of the output.  The token-major layout is
  timed beside it.
"""
from __future__ import annotations

import hashlib
import json
import os
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))

HBM_PEAK_GBS = 8000.0
MASK64 = (1 << 64) - 1  # fingerprints are unsigned; torch holds them as int64
BF16_MFMA_PEAK_TFLOPS = 2500.0
# fp32 vector operations, one per lane per cycle: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bitwise_deterministic_fp32_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}/{workload}")
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _log(msg):
    import sys
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _Timer:
    def __init__(self, torch, phases):
        self.torch, self.phases, self.events = torch, phases, []

    def step(self):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.phases) + 1)]
        self.events.append(evs)
        return evs

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in self.events])) for i, n in enumerate(self.phases)}


def _timed(torch, steps, fn):
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def graph_ms(torch, fn, steps: int, warmup: int) -> float:
    """Per-step time of fn captured once in a HIP graph and replayed `steps`
    times (the library's calls launch only kernels on the current stream, so
    they capture whole; the replays cost no host launch time)."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    ms = _timed(torch, steps, g.replay)
    del g
    return ms


def cold_ms(torch, fn, reps: int = 10, flush_mib: int = 1024) -> float:
    """Median time of one call with the caches cold: before each call an
    untimed read of 1 GiB (four times the 256 MB Infinity Cache) evicts L2
    and the Infinity Cache.  A read leaves no dirty lines behind, so nothing
    is written back during the timed call.  The start event is queued behind
    the read without waiting for it, so the host-side cost of the call (the
    Python binding, argument checks, the launch) overlaps the read and the
    events time the GPU work alone."""
    buf = torch.zeros(flush_mib << 18, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        buf.sum()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    return float(sorted(ts)[len(ts) // 2])


def cold_roofline(alg_bytes: int, ms: float) -> dict:
    """The roofline figures of one launch with cold caches."""
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"cold_cache_launch_ms": round(ms, 4), "achieved_cold_cache": round(gbs, 1),
            "frac_cold_cache": round(gbs / HBM_PEAK_GBS, 4)}


def run(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only=False):
    if name == "sparse_attn_dk_fused":
        return _fused_dk_main(torch, dr, steps, warmup, cpu_seconds, want_cpu, step_only)
    if name == "grouped_wgrad":
        return _grouped_wgrad(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only)
    if name in ("sparse_attn_dk", "embedding_grad"):
        return _index_add(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only)
    if name == "decode_attention":
        return _decode(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only)
    return _splitk(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only)


DECODE_KV_CHUNK = 512


def _decode_bytes(lens, Hq, Hkv, D, chunk):
    """Algorithmic bytes of one decode attention call: the K and V rows of every
    cached token, q, the private chunk partials (written, then read by the
    merge) and the output."""
    kv = int(lens.astype(np.int64).sum()) * Hkv * D * 2 * 2
    chunks = int(((lens.astype(np.int64) + chunk - 1) // chunk).sum())
    partials = chunks * Hq * (8 + D * 4)
    return kv + len(lens) * Hq * D * 2 + 2 * partials + len(lens) * Hq * D * 4


def _decode(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only):
    import oracle
    import workloads
    _log(f"{name}: generating inputs")
    inp = workloads.make(name)
    B, Lmax, Hq, Hkv, D, C = inp.B, inp.Lmax, inp.Hq, inp.Hkv, inp.D, DECODE_KV_CHUNK
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).cuda()
    k_tok = torch.from_numpy(inp.k.view(np.int16)).view(torch.bfloat16).cuda()
    v_tok = torch.from_numpy(inp.v.view(np.int16)).view(torch.bfloat16).cuda()
    k = k_tok.permute(0, 2, 1, 3).contiguous()   # head-major [B, Hkv, Lmax, D]
    v = v_tok.permute(0, 2, 1, 3).contiguous()
    lens = torch.from_numpy(inp.lens).cuda()
    out = torch.empty(B, Hq, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(dr.dr_decode_attention_workspace_size(B, Hq, Lmax, C), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fp = torch.empty(1, dtype=torch.int64, device="cuda")
    ws_fp = torch.empty(dr.dr_fingerprint_workspace_size(B * Hq * D * 4), dtype=torch.uint8, device="cuda")
    call_bytes = _decode_bytes(inp.lens, Hq, Hkv, D, C)
    step_bytes = call_bytes + B * Hq * D * 4
    timer = _Timer(torch, ["decode_attention", "fingerprint"])

    def call(chunk=C, o=out, w=ws, kk=k, vv=v, hm=True):
        dr.dr_decode_attention(q, kk, vv, lens, inp.scale, chunk, head_major=hm, out=o, ws=w, dev_status=status)

    def step(evs=None):
        if evs: evs[0].record()
        call()
        if evs: evs[1].record()
        dr.dr_fingerprint(out, out=fp, ws=ws_fp)
        if evs: evs[2].record()

    for _ in range(warmup):
        step()
    dr.dr_read_status(status)
    _log(f"{name}: timing {steps} steps")
    eager_ms = _timed(torch, steps, lambda: step(timer.step()))
    ph = timer.mean_ms()
    det_ms = ph["decode_attention"]
    h0 = int(fp.item())
    ms_step = graph_ms(torch, step, steps, warmup)
    if int(fp.item()) != h0:
        raise RuntimeError("graph replays of the decode step changed its output")
    extras, extra_roofline = {}, {}
    if not step_only:
        ms_cold = cold_ms(torch, call)
        legs = {}
        # the occupancy-chosen partition of a split-KV heuristic (batch-variant) on the same batch
        occ = dr.dr_decode_attention_occupancy_chunk(B, Hkv, Lmax)
        ws_o = torch.empty(dr.dr_decode_attention_workspace_size(B, Hq, Lmax, occ), dtype=torch.uint8,
                           device="cuda")
        o2 = torch.empty_like(out)
        for _ in range(warmup):
            call(occ, o2, ws_o)
        legs["occupancy_chunk"] = occ
        legs["occupancy_chunk_ms"] = round(_timed(torch, steps, lambda: call(occ, o2, ws_o)), 4)
        # the pages' long-prefix scheme: each (sequence, KV head) walked serially by one workgroup
        serial = ((Lmax + 63) // 64) * 64
        ws_s = torch.empty(dr.dr_decode_attention_workspace_size(B, Hq, Lmax, serial), dtype=torch.uint8,
                           device="cuda")
        for _ in range(warmup):
            call(serial, o2, ws_s)
        legs["one_workgroup_per_sequence_head_ms"] = round(_timed(torch, steps, lambda: call(serial, o2, ws_s)), 4)
        # the token-major layout of the same cache (same bits)
        for _ in range(warmup):
            call(C, o2, ws, k_tok, v_tok, False)
        legs["token_major_layout_ms"] = round(_timed(torch, steps, lambda: call(C, o2, ws, k_tok, v_tok, False)), 4)
        torch.cuda.synchronize()
        if not torch.equal(o2.view(torch.int32), out.view(torch.int32)):
            raise RuntimeError("token-major and head-major layouts gave different bits")
        # one long sequence alone: fixed chunks against the heuristic's choice for a batch of one
        L1 = int(inp.lens.max())
        b1 = int(np.argmax(inp.lens))
        q1, k1, v1 = q[b1:b1 + 1].contiguous(), k[b1:b1 + 1].contiguous(), v[b1:b1 + 1].contiguous()  # head-major
        l1 = lens[b1:b1 + 1].contiguous()
        o1 = torch.empty(1, Hq, D, dtype=torch.float32, device="cuda")
        occ1 = dr.dr_decode_attention_occupancy_chunk(1, Hkv, Lmax)
        for c1 in (C, occ1):
            w1 = torch.empty(dr.dr_decode_attention_workspace_size(1, Hq, Lmax, c1), dtype=torch.uint8,
                             device="cuda")
            for _ in range(warmup):
                dr.dr_decode_attention(q1, k1, v1, l1, inp.scale, c1, head_major=True, out=o1, ws=w1)
            legs[f"single_sequence_L{L1}_chunk{c1}_ms"] = round(
                _timed(torch, steps, lambda: dr.dr_decode_attention(q1, k1, v1, l1, inp.scale, c1, head_major=True,
                                                                    out=o1, ws=w1)), 4)
        extras = {"cold_cache_ms_per_call": round(ms_cold, 4), "partition_legs": legs,
                  "overhead_vs_occupancy_chunk": round(det_ms / legs["occupancy_chunk_ms"] - 1, 4)}
        extra_roofline = cold_roofline(call_bytes, ms_cold)
    achieved = call_bytes / (det_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": ms_step,
        "value": step_bytes / (ms_step * 1e-3) / 1e9,
        "timing": "step replayed from a HIP graph; eager_ms_per_step with HIP events between the calls",
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": f"{name}: {B} sequences, lengths U[1,{Lmax}] (total {int(inp.lens.sum())} tokens), "
                               f"{Hq} query / {Hkv} KV heads, head dim {D}, bf16 head-major KV cache "
                               f"[{B},{Hkv},{Lmax},{D}], fp32 output, KV chunk {C}",
                   "batch": B, "max_seq_len": Lmax, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "kv_chunk": C,
                   "kv_layout": "head-major",
                   "step": "dr_decode_attention (chunk partials + ordered merge) + fingerprint",
                   "step_algorithmic_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "dr_decode_attention call (decode_partial_kernel, decode_merge_kernel)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("dr_decode_attention", name, source_digest("decode.hip", "device.h")),
                     "algorithmic_bytes_per_launch": call_bytes, "avg_launch_ms": round(det_ms, 4),
                     **extra_roofline},
        "phases_ms": {k: round(v, 4) for k, v in ph.items()},
        **extras,
    }
    if want_cpu:
        res["cpu_baseline"] = _cpu_decode(oracle, inp, cpu_seconds)
    return res


def _cpu_decode(oracle, inp, seconds):
    """The oracle on the first sequences of the same batch, its numpy products
    held to one thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _cpu_decode_1(oracle, inp, seconds)


def _cpu_decode_1(oracle, inp, seconds):
    import dataclasses
    t0 = time.perf_counter()
    oracle.decode_attention(inp.q[:1], inp.k[:1], inp.v[:1], inp.lens[:1], inp.scale)
    dt = max(time.perf_counter() - t0, 1e-6)
    budget = seconds / dt * max(int(inp.lens[0]), 1)       # cached tokens the oracle gets through in `seconds`
    m = max(1, min(inp.B, int(np.searchsorted(np.cumsum(inp.lens), budget))))
    _log(f"cpu baseline: oracle decode attention on the first {m} of {inp.B} sequences")
    sub = dataclasses.replace(inp, B=m, q=inp.q[:m], k=inp.k[:m], v=inp.v[:m], lens=inp.lens[:m])
    t0 = time.perf_counter()
    oracle.decode_attention(sub.q, sub.k, sub.v, sub.lens, sub.scale)
    el = time.perf_counter() - t0
    kv = int(sub.lens.astype(np.int64).sum()) * inp.Hkv * inp.D * 4
    return {"value": round(kv / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} of {inp.B} sequences ({int(sub.lens.sum())} cached tokens), KV bytes only, "
                      f"{el:.1f} s", "seconds": round(el, 2)}


def _index_add(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only):
    import oracle
    import workloads
    _log(f"{name}: generating inputs")
    inp = workloads.make(name)
    D, H, n = inp.D, inp.H, inp.n
    index = torch.from_numpy(inp.index).cuda()
    src = torch.from_numpy(inp.src.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.from_numpy(inp.out0).cuda()
    counts = np.bincount(inp.index, minlength=D)
    touched = int((counts > 0).sum())
    red_bytes = n * H * 2 + n * 4 + 2 * touched * H * 4     # contributions, index, RMW of touched rows
    fp_bytes = D * H * 4
    step_bytes = red_bytes  # the fingerprint update reads nothing the reduction does not already hold
    ws = torch.empty(dr.dr_index_add_workspace_size(n, D, H), dtype=torch.uint8, device="cuda")
    fp = torch.empty(1, dtype=torch.int64, device="cuda")
    ws_fp = torch.empty(dr.dr_fingerprint_workspace_size(fp_bytes), dtype=torch.uint8, device="cuda")
    timer = _Timer(torch, ["index_add_fingerprinted"])
    dr.dr_fingerprint(out, out=fp, ws=ws_fp)  # the destination's fingerprint, kept current from here on

    def step(evs=None):
        if evs: evs[0].record()
        dr.dr_index_add_fingerprinted(out, src, index, fp, ws=ws)
        if evs: evs[1].record()

    for _ in range(warmup):
        step()
    dr.dr_workspace_status(ws)
    torch.cuda.synchronize()
    if int(fp.item()) & MASK64 != dr.fingerprint_value(out):
        raise RuntimeError("the incremental fingerprint differs from the fingerprint of the destination")
    _log(f"{name}: timing {steps} steps")
    eager_ms = _timed(torch, steps, lambda: step(timer.step()))
    ph = timer.mean_ms()
    det_ms = ph["index_add_fingerprinted"]
    ms_step = graph_ms(torch, step, steps, warmup)
    dr.dr_workspace_status(ws)
    torch.cuda.synchronize()
    if int(fp.item()) & MASK64 != dr.fingerprint_value(out):
        raise RuntimeError("the incremental fingerprint drifted during the graph replays")
    extras, extra_roofline = {}, {}
    if not step_only:
        ms_cold = cold_ms(torch, step)

        # the step with the plain call and a full fingerprint of the destination
        def full_step():
            dr.dr_index_add(out, src, index, ws=ws)
            dr.dr_fingerprint(out, out=fp, ws=ws_fp)

        for _ in range(warmup):
            full_step()
        ms_full = graph_ms(torch, full_step, steps, warmup)
        ms_plain = _timed(torch, steps, lambda: dr.dr_index_add(out, src, index, ws=ws))

        # reused plan: sort once, then only the plan + ordered reduction each step
        perm, seg, _ = dr.dr_sort_by_dest(index, D, want_inv=False)
        ws2 = torch.empty_like(ws)
        for _ in range(warmup):
            dr.dr_index_add(out, src, index, perm=perm, seg_offsets=seg, ws=ws2)
        ms_plan = _timed(torch, steps, lambda: dr.dr_index_add(out, src, index, perm=perm, seg_offsets=seg, ws=ws2))
        ws_sort = torch.empty(dr.dr_sort_workspace_size(n, D), dtype=torch.uint8, device="cuda")
        ms_sort = _timed(torch, steps, lambda: dr.dr_sort_by_dest(index, D, perm=perm, seg_offsets=seg, want_inv=False,
                                                                   ws=ws_sort))
        # atomic baseline on the same destination
        for _ in range(warmup):
            dr.dr_index_add_atomic(out, src, index)
        ms_atomic = _timed(torch, steps, lambda: dr.dr_index_add_atomic(out, src, index))
        # the pages' default path itself: torch's index_add_ (atomic adds), on fp32 rows converted beforehand
        # (index_add_ needs the destination's dtype), so it reads twice the bytes of the bf16 rows
        src32 = src.float()
        for _ in range(warmup):
            out.index_add_(0, index, src32)
        ms_torch = _timed(torch, steps, lambda: out.index_add_(0, index, src32))
        del src32

        fused = _fused_dk(torch, dr, steps, warmup, want_cpu, cpu_seconds) if name == "sparse_attn_dk" else None
        ia_cold = cold_ms(torch, lambda: dr.dr_index_add_fingerprinted(out, src, index, fp, ws=ws))
        extras = {
            "cold_cache_ms_per_step": round(ms_cold, 4),
            "plain_index_add_ms": round(ms_plain, 4),
            "step_with_full_fingerprint_ms": round(ms_full, 4),
            "reused_plan_ms": round(ms_plan, 4), "sort_only_ms": round(ms_sort, 4),
            "overhead_vs_atomic": {"deterministic_ms": round(ms_plain, 4), "atomic_ms": round(ms_atomic, 4),
                                   "torch_index_add_fp32_ms": round(ms_torch, 4),
                                   "overhead": round(ms_plain / min(ms_atomic, ms_torch) - 1, 4),
                                   "overhead_reused_plan": round(ms_plan / min(ms_atomic, ms_torch) - 1, 4),
                                   "note": "overhead against the faster of dr_index_add_atomic (bf16 rows, 16-byte "
                                           "loads) and torch index_add_ (fp32 rows)"},
        }
        if fused:
            extras["fused_dk"] = fused
        extra_roofline = cold_roofline(red_bytes, ia_cold)
    # the ordered reduction alone (segmented reduce + tile combine): events the library records around it
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for b_, e_ in pairs:
        dr.dr_set_phase_events(b_, e_)
        step()
    dr.dr_set_phase_events()
    torch.cuda.synchronize()
    red_ms = float(np.mean([b_.elapsed_time(e_) for b_, e_ in pairs]))
    achieved = red_bytes / (red_ms * 1e-3) / 1e9
    call_achieved = red_bytes / (det_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": ms_step,
        "value": step_bytes / (ms_step * 1e-3) / 1e9,
        "timing": "step replayed from a HIP graph; eager_ms_per_step with HIP events between the calls",
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": f"{name}: index_add of {n} bf16 rows of width {H} into {D} fp32 rows "
                               f"({touched} touched, longest segment {int(counts.max())})",
                   "n": n, "num_dests": D, "hidden": H, "touched_rows": touched,
                   "step": "dr_index_add_fingerprinted (sort + plan + ordered reduce + update, fingerprint kept "
                           "current from the rewritten rows)",
                   "step_algorithmic_bytes": step_bytes},
        "roofline": {"bound": "hbm",
                     "kernel": "segreduce_kernel + tilecombine_kernel (the ordered reduction of the call)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("segreduce+tilecombine", name,
                                                 source_digest("segreduce.hip", "lds_tile.h", "internal.h",
                                                               "device.h")),
                     "algorithmic_bytes_per_launch": red_bytes, "avg_launch_ms": round(red_ms, 4),
                     "timed_by": "events recorded by the library around the two kernels (dr_set_phase_events)",
                     "whole_call": {"kernel": "dr_index_add_fingerprinted (sort, plan, segreduce, tilecombine, "
                                              "fingerprint update)",
                                    "achieved": round(call_achieved, 1), "frac": round(call_achieved / HBM_PEAK_GBS, 4),
                                    "avg_launch_ms": round(det_ms, 4),
                                    "traffic": measured_traffic("dr_index_add_fingerprinted", name,
                                                                source_digest("sort.hip", "segreduce.hip",
                                                                              "lds_tile.h", "fingerprint.hip",
                                                                              "internal.h", "device.h")),
                                    **extra_roofline}},
        "phases_ms": {k: round(v, 4) for k, v in ph.items()},
        **extras,
    }
    if want_cpu:
        res["cpu_baseline"] = _cpu_index_add(oracle, inp, cpu_seconds)
    return res


def _fused_dk_main(torch, dr, steps, warmup, cpu_seconds, want_cpu, step_only):
    """The fused key gradient as the line's own workload (for profiling it
    alone): step_only times the call and nothing else."""
    import workloads
    if not step_only:
        r = _fused_dk(torch, dr, steps, warmup, want_cpu, cpu_seconds)
        ms = r.pop("ms")
        alg = r["algorithmic_bytes"]
        return {"ms_per_step": ms, "value": alg / (ms * 1e-3) / 1e9,
                "config": {"workload": "sparse_attn_dk_fused: dK[key] += fl32(dS[q,j] Q[q]) over the queries "
                                       "that selected the key; Q bf16 [8192,128], dS fp32 [8192,512], 65,536 keys"},
                **r}
    inp = workloads.sparse_attn_dk_inputs(workloads.CONFIGS["sparse_attn_dk"]["seed"])
    nq, topk = inp.key_idx.shape
    Q = torch.from_numpy(inp.Q.view(np.int16)).view(torch.bfloat16).cuda()
    dS = torch.from_numpy(inp.dS).cuda()
    idx = torch.from_numpy(inp.key_idx).cuda()
    dK = torch.from_numpy(inp.dK0).cuda()
    ws = torch.empty(dr.dr_sparse_attn_dk_workspace_size(nq, topk, inp.num_keys, inp.H), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        dr.dr_sparse_attn_dk(dK, Q, dS, idx, ws=ws)
    ms = _timed(torch, steps, lambda: dr.dr_sparse_attn_dk(dK, Q, dS, idx, ws=ws))
    touched = int((np.bincount(inp.key_idx.reshape(-1), minlength=inp.num_keys) > 0).sum())
    n = nq * topk
    alg = nq * inp.H * 2 + n * 4 + n * 4 + 2 * touched * inp.H * 4
    return {"ms_per_step": ms, "value": alg / (ms * 1e-3) / 1e9,
            "config": {"workload": "sparse_attn_dk_fused (step only)"},
            "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def _fused_dk(torch, dr, steps, warmup, want_cpu=False, cpu_seconds=4.0):
    """dr_sparse_attn_dk on the same key selection: the contributions
    fl32(dS * Q) are formed in the reduce instead of read as 1.07 GB of rows."""
    import oracle
    import workloads
    _log("sparse_attn_dk: fused key gradient (query rows and score gradients)")
    inp = workloads.sparse_attn_dk_inputs(workloads.CONFIGS["sparse_attn_dk"]["seed"])
    nq, topk = inp.key_idx.shape
    Q = torch.from_numpy(inp.Q.view(np.int16)).view(torch.bfloat16).cuda()
    dS = torch.from_numpy(inp.dS).cuda()
    idx = torch.from_numpy(inp.key_idx).cuda()
    dK = torch.from_numpy(inp.dK0).cuda()
    ws = torch.empty(dr.dr_sparse_attn_dk_workspace_size(nq, topk, inp.num_keys, inp.H), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        dr.dr_sparse_attn_dk(dK, Q, dS, idx, ws=ws)
    ms = _timed(torch, steps, lambda: dr.dr_sparse_attn_dk(dK, Q, dS, idx, ws=ws))
    perm, seg, _ = dr.dr_sort_by_dest(idx.reshape(-1), inp.num_keys, want_inv=False)
    for _ in range(warmup):
        dr.dr_sparse_attn_dk(dK, Q, dS, idx, perm=perm, seg_offsets=seg, ws=ws)
    ms_plan = _timed(torch, steps, lambda: dr.dr_sparse_attn_dk(dK, Q, dS, idx, perm=perm, seg_offsets=seg, ws=ws))
    # the ordered reduction alone, timed by the events the library records around it
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for b_, e_ in pairs:
        dr.dr_set_phase_events(b_, e_)
        dr.dr_sparse_attn_dk(dK, Q, dS, idx, ws=ws)
    dr.dr_set_phase_events()
    torch.cuda.synchronize()
    red_ms = float(np.mean([b_.elapsed_time(e_) for b_, e_ in pairs]))
    counts = np.bincount(inp.key_idx.reshape(-1), minlength=inp.num_keys)
    touched = int((counts > 0).sum())
    n = nq * topk
    alg = nq * inp.H * 2 + n * 4 + n * 4 + 2 * touched * inp.H * 4  # Q, dS, key ids, dK read-modify-write
    # The reduce forms each contribution element with three vector operations (widen the bf16 query
    # value, multiply by dS, add in the defined order); its bound is the vector ALU, one operation per
    # lane per cycle (no fused or packed forms: products are rounded before they are added).
    vops = n * inp.H * 3
    res = {"ms": round(ms, 4), "reused_plan_ms": round(ms_plan, 4), "algorithmic_bytes": alg,
           "roofline": {"bound": "alu", "kernel": "segreduce_gen16_kernel + tilecombine_kernel (contributions "
                                                  "formed from Q and the sorted dS)",
                        "achieved": round(vops / (red_ms * 1e-3) / 1e12, 2), "peak": VALU_PEAK_TOPS,
                        "unit": "Tops/s", "frac": round(vops / (red_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                        "vector_ops_per_launch": vops, "avg_launch_ms": round(red_ms, 4),
                        "traffic": measured_traffic("segreduce+tilecombine", "sparse_attn_dk_fused",
                                                    source_digest("segreduce.hip", "lds_tile.h", "internal.h",
                                                                  "device.h")),
                        "hbm_view": {"achieved": round(alg / (red_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(alg / (red_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                        "whole_call": {"achieved": round(vops / (ms * 1e-3) / 1e12, 2),
                                       "frac": round(vops / (ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4),
                                       "hbm_achieved_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                                       "avg_launch_ms": round(ms, 4)}},
           "note": "contributions formed from Q [8192,128] bf16 and dS [8192,512] fp32; the same key selection"}
    if want_cpu:
        # the oracle on the first queries of the same selection, one thread and the host's cores
        q = max(1, min(nq, int(nq * min(1.0, cpu_seconds / 8.0))))
        t0 = time.perf_counter()
        one = oracle.sparse_attn_dk(inp.dK0, inp.Q[:q], inp.dS[:q], inp.key_idx[:q])
        el = time.perf_counter() - t0
        th = host_threads()
        t0 = time.perf_counter()
        many = oracle.sparse_attn_dk(inp.dK0, inp.Q[:q], inp.dS[:q], inp.key_idx[:q], threads=th)
        el_mt = time.perf_counter() - t0
        same = bool(np.array_equal(one.view(np.uint32), many.view(np.uint32)))
        if not same:
            raise RuntimeError("the oracle's bits changed with its thread count")
        per_q = inp.H * 2 + topk * 8
        res["cpu_baseline"] = {"value": round(per_q * q / el_mt / 1e9, 4), "unit": "GB/s", "cores": th,
                               "kind": "oracle",
                               "sample": f"first {q} of {nq} queries; {th} threads {el_mt:.1f} s, 1 thread {el:.1f} s",
                               "seconds": round(el_mt, 2),
                               "single_thread": {"value": round(per_q * q / el / 1e9, 4), "cores": 1,
                                                 "seconds": round(el, 2)},
                               "bits_identical_across_thread_counts": same}
    return res


def host_threads() -> int:
    """Host threads for the oracle's multi-threaded timing: the CPU share of one GPU (16) at most."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_index_add(oracle, inp, seconds):
    """The oracle on the first contributions of the same workload (a prefix of the batch), on one thread and
    on the host's cores (destination ranges per thread; the bits must not change)."""
    n, H = inp.n, inp.H
    per_row = H * 2 + 4
    m = min(n, 4096)
    t0 = time.perf_counter()
    oracle.index_add(inp.out0, inp.src[:m], inp.index[:m])
    dt = max(time.perf_counter() - t0, 1e-6)
    # the full-destination copy and sort dominate small prefixes; scale linearly as an estimate
    m2 = int(min(n, m * max(1.0, seconds / dt)))
    _log(f"cpu baseline: oracle index_add on the first {m2} of {n} contributions")
    t0 = time.perf_counter()
    one = oracle.index_add(inp.out0, inp.src[:m2], inp.index[:m2])
    el = time.perf_counter() - t0
    th = host_threads()
    t0 = time.perf_counter()
    many = oracle.index_add(inp.out0, inp.src[:m2], inp.index[:m2], threads=th)
    el_mt = time.perf_counter() - t0
    same = bool(np.array_equal(one.view(np.uint32), many.view(np.uint32)))
    if not same:
        raise RuntimeError("the oracle's bits changed with its thread count")
    return {"value": round(per_row * m2 / el_mt / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
            "sample": f"first {m2} of {n} contributions of the same workload; {th} threads {el_mt:.1f} s, "
                      f"1 thread {el:.1f} s",
            "seconds": round(el_mt, 2),
            "single_thread": {"value": round(per_row * m2 / el / 1e9, 4), "cores": 1, "seconds": round(el, 2)},
            "bits_identical_across_thread_counts": same}


def _grouped_wgrad(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only):
    import oracle
    import workloads
    _log(f"{name}: generating inputs")
    inp = workloads.grouped_wgrad_inputs(1002)
    K, M, N, S = inp.K, inp.M, inp.N, inp.split_tokens
    G = inp.group_offsets.size - 1
    X = torch.from_numpy(inp.X.view(np.int16)).view(torch.bfloat16).cuda()
    dY = torch.from_numpy(inp.dY.view(np.int16)).view(torch.bfloat16).cuda()
    off = torch.from_numpy(inp.group_offsets).cuda()
    out = torch.empty(G, M, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(dr.dr_grouped_wgrad_workspace_size(K, G, S, M, N), dtype=torch.uint8, device="cuda")
    flops = 2 * K * M * N
    hbm_bytes = K * M * 2 + K * N * 2 + G * M * N * 4  # X and dY read once, dW written once

    def step():
        dr.dr_grouped_wgrad(X, dY, off, S, out=out, ws=ws)

    for _ in range(warmup):
        step()
    dr.dr_workspace_status(ws)
    h0 = dr.fingerprint_value(out)
    _log(f"{name}: timing {steps} steps")
    eager_ms = _timed(torch, steps, step)
    ms_step = graph_ms(torch, step, steps, warmup)
    if dr.fingerprint_value(out) != h0:
        raise RuntimeError("replays of the grouped weight gradient changed its output")
    tflops = flops / (eager_ms * 1e-3) / 1e12
    extras = {}
    if not step_only:
        # the same result through materialised slot partials: the thin-N split-K tiles, then the reduce
        Pg, so, wsg = dr.dr_grouped_splitk_gemm_tn(X, dY, off, S)

        def materialised():
            dr.dr_grouped_splitk_gemm_tn(X, dY, off, S, partials=Pg, slot_offsets=so, ws=wsg)
            return dr.dr_grouped_splitk_reduce(Pg, so, wsg)
        ref = materialised()
        if dr.fingerprint_value(ref) != h0:
            raise RuntimeError("the register-slot and materialised-partial paths differ")
        ms_mat = _timed(torch, 2, materialised)
        del Pg, ref
        torch.cuda.empty_cache()
        # a library GEMM per expert (hipBLASLt through torch, bf16 out, no slots): context for the MFMA rate
        Xt = [X[int(inp.group_offsets[g]):int(inp.group_offsets[g + 1])].t().contiguous() for g in range(G)]
        dYg = [dY[int(inp.group_offsets[g]):int(inp.group_offsets[g + 1])] for g in range(G)]

        def library():
            for g in range(G):
                torch.matmul(Xt[g], dYg[g])
        for _ in range(warmup):
            library()
        ms_lib = _timed(torch, steps, library)
        del Xt, dYg
        extras = {
            "materialised_partials_ms": round(ms_mat, 4),
            "library_gemm_per_expert_ms": round(ms_lib, 4),
            "library_gemm_tflops": round(flops / (ms_lib * 1e-3) / 1e12, 1),
            "library_note": "torch.matmul of each expert's pre-transposed X rows with dY (hipBLASLt, bf16 output, "
                            "one GEMM per expert, no private slots); the transposes are outside the timing",
        }
    res = {
        "ms_per_step": ms_step,
        "value": tflops,
        # this line's value is MFMA work, not bytes
        "metric": "grouped weight gradient bf16 MFMA TFLOP/s (private token slots merged in slot order)",
        "unit": "TFLOP/s",
        "dtype": "bf16 products, f32 accumulation",
        "timing": "step replayed from a HIP graph; the roofline uses the eager per-call time",
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": f"{name}: dW[g] = X_g^T dY_g for the {G} hottest experts of the MoE routing "
                               f"(token counts {np.diff(inp.group_offsets).tolist()}), M {M}, N {N}, "
                               f"private slots of {S} tokens merged in slot order",
                   "K": K, "M": M, "N": N, "groups": G, "split_tokens": S, "flops": flops},
        "roofline": {"bound": "mfma", "kernel": "wgrad_kernel (with its plan and merge launches)",
                     "achieved": round(tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("wgrad_kernel", name,
                                                 source_digest("wgrad.hip", "lds_tile.h", "device.h")),
                     "algorithmic_flops_per_launch": flops, "hbm_algorithmic_bytes": hbm_bytes,
                     "avg_launch_ms": round(eager_ms, 4)},
        **extras,
    }
    if want_cpu:
        # the oracle's fp64 reference of the first expert's product on a sample of X's columns
        a, b = int(inp.group_offsets[0]), int(inp.group_offsets[1])
        cols = 8
        t0 = time.perf_counter()
        oracle.splitk_reference(np.ascontiguousarray(inp.X[a:b, :cols]), inp.dY[a:b])
        dt = max(time.perf_counter() - t0, 1e-6)
        cols = int(min(M, cols * max(1.0, cpu_seconds / dt)))
        Xs = np.ascontiguousarray(inp.X[a:b, :cols])
        t0 = time.perf_counter()
        oracle.splitk_reference(Xs, inp.dY[a:b])
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(2 * (b - a) * cols * N / el / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"fp64 reference of expert 0's product on {cols} of {M} columns, {el:.1f} s",
                               "seconds": round(el, 2)}
    return res


def _splitk(torch, dr, name, steps, warmup, cpu_seconds, want_cpu, step_only):
    import oracle
    import workloads
    _log(f"{name}: generating inputs")
    inp = workloads.make(name)
    K, M, N, S = inp.K, inp.M, inp.N, inp.splits
    X = torch.from_numpy(inp.X.view(np.int16)).view(torch.bfloat16).cuda()
    dY = torch.from_numpy(inp.dY.view(np.int16)).view(torch.bfloat16).cuda()
    partials = torch.empty(S, M, N, dtype=torch.float32, device="cuda")
    dW = torch.empty(M, N, dtype=torch.float32, device="cuda")
    fp = torch.empty(1, dtype=torch.int64, device="cuda")
    ws_rf = torch.empty(dr.dr_splitk_reduce_fingerprinted_workspace_size(S, M * N), dtype=torch.uint8,
                        device="cuda")
    gemm_bytes = K * M * 2 + K * N * 2 + S * M * N * 4
    red_bytes = S * M * N * 4 + M * N * 4
    # the reduce hashes dW as it stores it: the fingerprint reads nothing more
    step_bytes = gemm_bytes + red_bytes
    flops = 2 * K * M * N
    timer = _Timer(torch, ["splitk_gemm", "splitk_reduce"])

    def step(evs=None):
        if evs: evs[0].record()
        dr.dr_splitk_gemm_tn(X, dY, S, partials=partials)
        if evs: evs[1].record()
        dr.dr_splitk_reduce_fingerprinted(partials, fp, out=dW, ws=ws_rf)
        if evs: evs[2].record()

    for _ in range(warmup):
        step()
    _log(f"{name}: timing {steps} steps")
    eager_ms = _timed(torch, steps, lambda: step(timer.step()))
    ph = timer.mean_ms()
    g_ms = ph["splitk_gemm"]
    h0 = int(fp.item())
    ms_step = graph_ms(torch, step, steps, warmup)
    if int(fp.item()) != h0:
        raise RuntimeError("graph replays of the split-K step changed its output")
    det_ms = ph["splitk_gemm"] + ph["splitk_reduce"]
    extras, extra_roofline = {}, {}
    if not step_only:
        ms_cold = cold_ms(torch, step)
        dW_a = torch.empty_like(dW)
        atimer = _Timer(torch, ["zero", "splitk_gemm_atomic"])

        def astep(evs=None):
            if evs: evs[0].record()
            dW_a.zero_()
            if evs: evs[1].record()
            dr.dr_splitk_gemm_tn_atomic(X, dY, S, out=dW_a)
            if evs: evs[2].record()

        for _ in range(warmup):
            astep()
        for _ in range(steps):
            astep(atimer.step())
        aph = atimer.mean_ms()
        # the single-pass alternative: one split, so one workgroup per 64-column M tile walks all K tokens
        p1 = torch.empty(1, M, N, dtype=torch.float32, device="cuda")
        for _ in range(warmup):
            dr.dr_splitk_gemm_tn(X, dY, 1, partials=p1)
        ms_nosplit = _timed(torch, steps, lambda: dr.dr_splitk_gemm_tn(X, dY, 1, partials=p1))
        # the grouped form of the same contraction: 16 unequal groups (expert-like sizes), slots of 256 tokens
        sizes = np.array([int(K * w) for w in np.linspace(2.0, 0.05, 16) / np.linspace(2.0, 0.05, 16).sum()])
        sizes[0] += K - sizes.sum()
        offs = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)).cuda()
        Pg, so, wsg = dr.dr_grouped_splitk_gemm_tn(X, dY, offs, 256)
        dWg = dr.dr_grouped_splitk_reduce(Pg, so, wsg)

        def grouped():
            dr.dr_grouped_splitk_gemm_tn(X, dY, offs, 256, partials=Pg, slot_offsets=so, ws=wsg)
            dr.dr_grouped_splitk_reduce(Pg, so, wsg, out=dWg)

        for _ in range(warmup):
            grouped()
        ms_grouped = _timed(torch, steps, grouped)
        dr.dr_workspace_status(wsg)
        g_cold = cold_ms(torch, lambda: dr.dr_splitk_gemm_tn(X, dY, S, partials=partials))
        at_ms = aph["zero"] + aph["splitk_gemm_atomic"]
        extras = {
            "overhead_vs_atomic": {"deterministic_ms": round(det_ms, 4), "atomic_zero_plus_gemm_ms": round(at_ms, 4),
                                   "overhead": round(det_ms / at_ms - 1, 4)},
            "cold_cache_ms_per_step": round(ms_cold, 4),
            "no_split_ms": round(ms_nosplit, 4),
            "grouped_16_groups_ms": round(ms_grouped, 4),
        }
        extra_roofline = cold_roofline(gemm_bytes, g_cold)
    achieved = gemm_bytes / (g_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": ms_step,
        "value": step_bytes / (ms_step * 1e-3) / 1e9,
        "timing": "step replayed from a HIP graph; eager_ms_per_step with HIP events between the calls",
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": f"{name}: dW = X^T dY, X bf16 [{K},{M}], dY bf16 [{K},{N}], {S} splits",
                   "K": K, "M": M, "N": N, "splits": S,
                   "step": "MFMA partials + ordered split reduce hashing dW as it stores it (the splitk_reduce "
                           "phase includes the fingerprint)", "step_algorithmic_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "splitk_stream_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("splitk_stream_kernel", name,
                                                 source_digest("splitk.hip", "lds_tile.h", "device.h")),
                     "algorithmic_bytes_per_launch": gemm_bytes, "avg_launch_ms": round(g_ms, 4),
                     **extra_roofline,
                     "headline": "cold-cache fraction: X (235 MB) fits the 256 MB Infinity Cache, so back-to-back "
                                 "launches are partly served by it",
                     "mfma_tflops": round(flops / (g_ms * 1e-3) / 1e12, 2),
                     "mfma_frac_of_bf16_peak": round(flops / (g_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 5)},
        "phases_ms": {k: round(v, 4) for k, v in ph.items()},
        **extras,
    }
    if want_cpu:
        t0 = time.perf_counter()
        cols = 64
        oracle.splitk_reference(inp.X[:, :cols].copy(), inp.dY)
        dt = time.perf_counter() - t0
        cols = int(min(M, cols * max(1.0, cpu_seconds / max(dt, 1e-6))))
        _log(f"cpu baseline: oracle split-K reference on {cols} of {M} columns")
        Xs = np.ascontiguousarray(inp.X[:, :cols])
        t0 = time.perf_counter()
        oracle.splitk_reference(Xs, inp.dY)
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round((K * cols * 2 + K * N * 2) / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{cols} of {M} columns of X (fp64 reference), {el:.1f} s",
                               "seconds": round(el, 2)}
    return res
