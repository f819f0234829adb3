"""Benchmark of the context-parallel attention hot path on one MI355X.

Headline (``value``): one rank's ring pass of the Wan2.2-shaped workload (10 heads of
128, S = 32768 over cp = 8, local 4096 queries): 8 online-max steps, every K/V chunk after
the rank's own moved into a receive buffer (the ring hop; each step carries the hop of the
chunk two steps ahead), then the LSE merge. value = algorithmic TFLOP/s of the whole pass
(4*H*Sq*S*D flops), inputs resident in HBM when timing starts.

Also reported (``workloads``): the const-max ring on the 720p share (40 heads,
local 9450), the striped causal ring at S = 128k (all 8 ranks' passes), DCP decode
over two interleaved paged shards (KV GB/s), and the tiny fp32 ring.

``roofline`` is measured live for the dominant kernel, the step kernel: 30 back-to-back
launches with the pass's inputs and workspace on one stream, bracketed by HIP events on that
stream (inside the pass the steps overlap on two streams, so their own durations include the
sharing). ``--roofline-only`` runs just that loop, for a profiler run of the kernel alone.
``cpu_baseline`` times the fp64 oracle on a bounded row sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu-baseline]
                       [--only constmax,striped,decode,tiny,copy] [--roofline-only]

The default warm-up is 50 passes (about 45 ms): after 3 the device has not reached its
steady clock and the same 20 passes take 9% longer.

``--only`` runs the headline plus the named extra workloads; ``copy`` times a plain device
copy of 1 GiB through the library (kv_chunk_copy), the reference used to scale the
FETCH_SIZE / WRITE_SIZE hardware counters into bytes.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


# HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch),
# scaled by the plain-copy calibration: the copy kernel moving 2 GiB in and 2 GiB out read
# FETCH_SIZE = 1048599.6 KiB and WRITE_SIZE = 2097263.8 KiB, so fetch x 2.0, write x 1.0.
# Each entry holds for the kernel source whose sha256 prefix it names; after an edit of that
# source the figure no longer describes the kernel and traffic is reported as null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {
    "attn_step_bf16/wan22_cp8_online": {"source": "attn_bf16.hip", "sha256": "82ac9e615e4caf61",
                                        "fetch_kib": 58130.2, "write_kib": 64920.0},
    "dcp_decode/dcp_decode_gqa": {"source": "decode.hip", "sha256": "2a888486a0688b34",
                                  "fetch_kib": 2774629.6 + 22236.4, "write_kib": 47159.9 + 1040.0},
}


def traffic(key):
    import hashlib
    t = TRAFFIC[key]
    path = os.path.join(ROOT, "context_attention_lse_amd", "csrc", t["source"])
    with open(path, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != t["sha256"]:
            return None
    return round((t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ring_flops(H, Sq, Sk, D):
    return 4.0 * H * Sq * Sk * D


def time_ring(rp, steps, warmup, torch, union=None):
    """Runs warmup + timed ring passes; returns (ms per pass, per-step mean kernel ms). The
    pass time comes from one event pair around ``steps`` passes with nothing else recorded;
    per-step durations (and, if ``union`` is a list, the mean span from the first step's
    start to the last step's end) come from a second, separately timed set of passes."""
    cp = rp.cp
    for _ in range(warmup):
        rp.run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(steps):
        rp.run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    n = max(2, min(steps, 5))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cp)]
          for _ in range(n)]
    for k in range(n):
        rp.run(timing_events=ev[k])
    torch.cuda.synchronize()
    per_step = [sum(ev[k][s][0].elapsed_time(ev[k][s][1]) for k in range(n)) / n for s in range(cp)]
    if union is not None:
        union.append(sum(max(ev[k][0][0].elapsed_time(ev[k][j][1]) for j in range(cp)) for k in range(n)) / n)
    return ms, per_step


def step_roofline(q, k, v, ws, torch, ca, reps=30):
    """Mean duration of the step kernel alone: ``reps`` back-to-back launches of
    ring_attn_step on the current stream with the headline's inputs and launch
    configuration (key-split workspace), bracketed by one HIP event pair."""
    B, Sq, H, D = q.shape
    o = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    ca.ring_attn_step(q, k, v, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ca.ring_attn_step(q, k, v, out=o, lse=lse, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def headline(args, torch, ca, workloads, gen, dev):
    wl = workloads.workload("wan22_cp8_online")
    log(f"[bench] generating {wl.name} inputs")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    del t
    # key-split steps on two compute streams, so one step's drain overlaps the next step's
    # start; each step carries the hop of the chunk two steps ahead on the CUs it leaves free
    rp = ca.ring.RingPass(q, kp, vp, 0, layout=wl.layout, variant="online", split=True, compute_streams=2,
                          fused_hops=True)
    Sq = wl.local_S
    flops_pass = ring_flops(wl.H, Sq, wl.S, wl.D)
    flops_step = ring_flops(wl.H, Sq, wl.local_S, wl.D)
    out = {"wl": wl, "inputs": (q, kp, vp)}
    if not args.roofline_only:
        log("[bench] timing ring pass")
        union = []
        ms, per_step = time_ring(rp, args.steps, args.warmup, torch, union)
        out.update({"ms": ms, "tflops": flops_pass / (ms * 1e-3) / 1e12,
                    "per_step_ms": per_step, "step_ms": sum(per_step) / len(per_step),
                    "steps_union_tflops": round(8 * flops_step / (union[0] * 1e-3) / 1e12, 2)})
    log("[bench] timing the step kernel alone (roofline)")
    kernel_ms = step_roofline(q, kp[0], vp[0], rp.ws[0], torch, ca)
    achieved = flops_step / (kernel_ms * 1e-3) / 1e12
    out["kernel_ms"] = kernel_ms
    out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                       "traffic": traffic("attn_step_bf16/wan22_cp8_online"),
                       "kernel": "attn_step_bf16 (ring_attn_step, key-split schedule)",
                       "per_launch": f"{flops_step / 1e9:.2f} GFLOP = 4*H*Sq*Sk*D, H=10 Sq=Sk=4096 D=128",
                       "kernel_ms": round(kernel_ms, 4),
                       "note": ("mean of 30 back-to-back launches on one stream with the pass's inputs and "
                                "workspace; inside the pass, steps alternate two streams and overlap")}
    return out


def cpu_baseline(q, kp, vp, D, budget_s=12.0):
    """fp64 oracle on a bounded sample of query rows (all heads, full key range)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    H = q.shape[2]
    scale = oracle.default_scale(D)
    S = kp.shape[0] * kp.shape[2]
    k_all = oracle.to_f64(kp[:, 0].reshape(S, H, D))
    v_all = oracle.to_f64(vp[:, 0].reshape(S, H, D))
    rng = np.random.default_rng(0)
    rows_done, t_total, batch = 0, 0.0, 32
    while t_total < budget_s and rows_done < q.shape[1]:
        rows = rng.choice(q.shape[1], size=batch, replace=False)
        qs = oracle.to_f64(q[0, rows])
        t0 = time.perf_counter()
        for h in range(H):
            oracle.attention(qs[:, h], k_all[:, h], v_all[:, h], scale)
        t_total += time.perf_counter() - t0
        rows_done += batch
    flops = ring_flops(H, rows_done, S, D)
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} query rows x {H} heads against all {S} keys (fp64 numpy oracle, "
                      f"{t_total:.1f} s); same per-row work as the GPU pass"}


def run_constmax(args, torch, ca, workloads, gen, dev):
    wl = workloads.workload("wan22_720p_constmax")
    log(f"[bench] {wl.name}")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout).contiguous()
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    del t
    out = {}
    for variant in ("constmax", "constmax_sinks", "online"):
        if variant == "constmax_sinks":
            # sink-robust pass (theta 4): on these QK-normed keys no key qualifies, so this
            # measures what the sink prologue, the per-tile sink test and the sink merge cost
            rp = ca.ring.RingPass(q, kp, vp, 0, variant="constmax", sink_theta=4.0)
            ms, _ = time_ring(rp, max(2, args.steps // 4), 1, torch)
            fl = ring_flops(wl.H, wl.local_S, wl.S, wl.D)
            out[variant] = {"ms_per_pass": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                            "sinks_found": int(rp.sinks["sink_cnt"].sum().item())}
            del rp
            continue
        # const-max steps carry their hops (2.8% faster on this share); the online pass keeps the
        # copy stream (its unsplit steps on two streams lost 0.9% with carried hops)
        rp = ca.ring.RingPass(q, kp, vp, 0, variant=variant, fused_hops=(variant == "constmax"))
        union = []
        ms, per_step = time_ring(rp, max(2, args.steps // 4), 1, torch, union)
        fl = ring_flops(wl.H, wl.local_S, wl.S, wl.D)
        step_ms = sum(per_step) / len(per_step)
        step_fl = ring_flops(wl.H, wl.local_S, wl.local_S, wl.D)
        ach = step_fl / (step_ms * 1e-3) / 1e12
        streams = 1 if rp.aux_stream is None else 2
        out[variant] = {"ms_per_pass": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                        "steps_union_tflops": round(wl.cp * step_fl / (union[0] * 1e-3) / 1e12, 2),
                        "compute_streams": streams}
        if streams == 1:
            out[variant].update({"step_kernel_ms": round(step_ms, 4), "step_tflops": round(ach, 2),
                                 "frac_bf16_peak": round(ach / PEAK_BF16_TFLOPS, 4)})
        else:
            # on two streams a step's events also span the neighbour step running beside it
            out[variant].update({"step_span_ms": round(step_ms, 4),
                                 "note": "steps alternate two streams and overlap: step_span_ms is each "
                                         "step's event span, not its kernel time; steps_union_tflops "
                                         "is the rate over the union of the step spans"})
        if variant == "constmax":
            # bound prologue: |k|^2 max over all 8 chunks + c for every query row (HBM-bound)
            ms_b = time_calls(rp.prologue, 10, torch)
            nbytes = (kp.numel() + q.numel()) * kp.element_size() + q.shape[1] * wl.H * 4
            out["bound"] = {"ms": round(ms_b, 4), "bytes": nbytes, "GBps": round(nbytes / (ms_b * 1e-3) / 1e9, 1),
                            "frac_hbm_peak": round(nbytes / (ms_b * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        else:
            # the 8-way merge of the online partials (HBM-bound: 8 x 193.5 MB in, 195 MB out)
            parts_o, parts_l = rp.o_parts[:wl.cp], rp.lse_parts[:wl.cp]
            ms_m = time_calls(lambda: ca.lse_merge(parts_o, parts_l, out=rp.out, lse_out=rp.lse), 10, torch)
            nbytes = (parts_o.numel() + parts_l.numel()) * 4 + (rp.out.numel() + rp.lse.numel()) * 4
            out["merge"] = {"ms": round(ms_m, 4), "bytes": nbytes, "GBps": round(nbytes / (ms_m * 1e-3) / 1e9, 1),
                            "frac_hbm_peak": round(nbytes / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del rp
    return {"workload": wl.name, "config": f"B=1 H=40 D=128 S=75600 cp=8 local=9450 bf16", **out}


def time_calls(fn, reps, torch):
    """Mean ms per call of ``fn`` (launches on the current stream), after one warm-up call."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_striped(args, torch, ca, workloads, gen, dev):
    wl = workloads.workload("striped_causal_128k")
    log(f"[bench] {wl.name}")
    t = gen.ring_inputs(wl, dev)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, "striped")
    vp = ca.ring.chunk_pool(t["v"], wl.cp, "striped")
    qs = [ca.ring.shard(t["q"], wl.cp, r, "striped").contiguous() for r in range(wl.cp)]
    del t
    copy_stream = torch.cuda.Stream()
    per_rank = []
    step_ms_all = []
    for r in range(wl.cp):
        rp = ca.ring.RingPass(qs[r], kp, vp, r, layout="striped", causal=True, copy_stream=copy_stream)
        ms, per_step = time_ring(rp, max(1, args.steps // 10), 1, torch)
        per_rank.append(ms)
        step_ms_all.extend(per_step)
        del rp
    S, H, D = wl.S, wl.H, wl.D
    total = 4.0 * H * D * S * (S + 1) / 2
    tot_ms = sum(per_rank)
    mean = tot_ms / len(per_rank)
    return {"workload": wl.name, "config": "B=1 H=32 D=128 S=131072 cp=8 striped causal bf16, all 8 ranks",
            "ms_all_ranks": round(tot_ms, 3), "tflops": round(total / (tot_ms * 1e-3) / 1e12, 2),
            "per_rank_ms": [round(x, 3) for x in per_rank],
            "rank_balance_max_over_mean": round(max(per_rank) / mean, 4),
            "mean_step_kernel_ms": round(sum(step_ms_all) / len(step_ms_all), 4)}


def run_decode(args, torch, ca, workloads, gen, dev):
    wl = workloads.workload("dcp_decode_gqa")
    log(f"[bench] {wl.name}: building paged shards")
    d = gen.decode_inputs(wl, dev)
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, wl.shards,
                                       wl.interleave, wl.block_size, d["block_rand"]) for r in range(wl.shards)]
    del d["k_seq"], d["v_seq"]
    run = ca.dcp.DcpDecode(d["q"], shards)
    steps = max(5, args.steps)
    for _ in range(2):
        run.run()
    torch.cuda.synchronize()
    kv_bytes = sum(sc.nbytes_kv for sc in shards)
    cs = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in shards]
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(steps):
        for r, sc in enumerate(shards):
            ev[k][r][0].record(cs)
            ca.dcp_decode_partial(run.q, sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens,
                                  out=run.o_parts[r], lse=run.lse_parts[r], workspace=run.ws[r])
            ev[k][r][1].record(cs)
        ca.lse_merge(run.o_parts, run.lse_parts, out=run.out, lse_out=run.lse)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    shard_ms = [sum(ev[k][r][0].elapsed_time(ev[k][r][1]) for k in range(steps)) / steps for r in range(len(shards))]
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    per_launch = [sc.nbytes_kv / (m * 1e-3) / 1e9 for sc, m in zip(shards, shard_ms)]
    ach = sum(per_launch) / len(per_launch)
    # the same step with a current token: the caches hold positions [0, N) of each sequence
    # and the new token at position N joins on its owner shard only (dcp_active_mask)
    prior = torch.tensor([int(n) for n in d["ctx"]], dtype=torch.int32, device=dev)
    k_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 21, dev, torch.bfloat16)
    v_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 22, dev, torch.bfloat16)
    ms_active = time_calls(lambda: run.run_active(prior, k_cur, v_cur, wl.interleave), steps, torch)
    return {"workload": wl.name, "config": "B=32 Hq=64 Hkv=8 D=128 bf16, ctx U[32k,128k], block 16, 2 interleaved shards",
            "kv_bytes": kv_bytes, "ms_per_step": round(ms, 4), "kv_GBps": round(gbs, 1),
            "with_current_token": {"ms_per_step": round(ms_active, 4),
                                   "kv_GBps": round(kv_bytes / (ms_active * 1e-3) / 1e9, 1),
                                   "note": "N resident tokens on their shards plus a new token at position N, attended on its owner shard only"},
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic("dcp_decode/dcp_decode_gqa"),
                         "kernel": "dcp_decode_split_kernel + combine (dcp_decode_partial)",
                         "per_launch": "one shard's resident K+V bytes = local tokens * Hkv * D * 2 * 2"}}


def run_prefill(args, torch, ca, workloads, gen, dev):
    """DCP prefill of one chunk (segmented attention on every rank + the LSE merge):
    S = 8192 new tokens after 65536 prior ones, 32 query heads over 8 KV heads, D = 128,
    DCP = 2 ranks interleaving blocks of 16, bf16; synthetic N(0, 1) inputs."""
    import numpy as np
    S, P, Hq, Hkv, D, W, I = 8192, 65536, 32, 8, 128, 2, 16
    log("[bench] dcp prefill")
    q = gen.normal((1, S, Hq, D), 901, dev, torch.bfloat16)
    k_all = gen.normal((P + S, Hkv, D), 902, dev, torch.bfloat16)
    v_all = gen.normal((P + S, Hkv, D), 903, dev, torch.bfloat16)
    offsets = np.array([0, P])
    caches = [ca.dcp.build_shard_cache(k_all, v_all, offsets, np.array([P]), r, W, I, 16) for r in range(W)]
    run = ca.dcp.DcpPrefill(q, k_all[P:].unsqueeze(0), v_all[P:].unsqueeze(0), caches, P, I)
    del k_all, v_all
    ms = time_calls(run.run, max(3, args.steps // 4), torch)
    flops = 4.0 * Hq * D * (S * P + S * (S + 1) / 2)
    return {"workload": "dcp_prefill_chunk", "config": f"S={S} after {P} prior, Hq={Hq} Hkv={Hkv} D={D}, DCP={W} "
            f"interleave {I}, bf16, both ranks + merge", "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def run_tiny(args, torch, ca, workloads, gen, dev):
    wl = workloads.workload("tiny_ring_fp32")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout).contiguous()
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    res = {"workload": wl.name, "config": "B=1 H=2 D=64 S=512 cp=4 fp32"}
    for variant in ("online", "constmax"):
        rp = ca.ring.RingPass(q, kp, vp, 0, variant=variant)
        ms, _ = time_ring(rp, 10, 2, torch)
        res[f"{variant}_ms_per_pass"] = round(ms, 4)
    return res


def run_copy(args, torch, ca, workloads, gen, dev):
    n = 1 << 29                      # 2**29 bf16 = 1 GiB per tensor
    src_k = torch.empty(n, dtype=torch.bfloat16, device=dev)
    src_v = torch.empty(n, dtype=torch.bfloat16, device=dev)
    dst_k = torch.empty_like(src_k)
    dst_v = torch.empty_like(src_v)
    src_k.zero_(); src_v.zero_()
    ca.kv_chunk_copy(dst_k, dst_v, src_k, src_v)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        ca.kv_chunk_copy(dst_k, dst_v, src_k, src_v)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    nbytes = 4 * n * 2                # read 2 GiB + write 2 GiB per call
    return {"workload": "device copy 2 x 1 GiB", "ms_per_call": round(ms, 4),
            "bytes_read_per_call": 2 * n * 2, "bytes_written_per_call": 2 * n * 2,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


EXTRAS = {"constmax": run_constmax, "striped": run_striped, "decode": run_decode, "prefill": run_prefill,
          "tiny": run_tiny, "copy": run_copy}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--roofline-only", action="store_true",
                    help="time only the step kernel's back-to-back launches (for profiling it alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="constmax,striped,decode,prefill,tiny",
                    help="comma-separated extra workloads to run after the headline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share only: the ring's other ranks are simulated on the same "
              "device, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import context_attention_lse_amd as ca
    import workloads
    from workloads import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ca._lib.load()

    h = headline(args, torch, ca, workloads, gen, dev)
    wl = h["wl"]
    if args.roofline_only:
        print(json.dumps({"workload": wl.name, "roofline": h["roofline"]}), flush=True)
        return
    line = {
        "metric": "ring-step attention TFLOP/s (% bf16 MFMA peak); DCP decode KV GB/s (% HBM)",
        "value": round(h["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded torch.randn; Q,K RMS-normalised across 40 heads x 128, gain 1)",
        "config": {"workload": wl.name, "B": wl.B, "heads": wl.H, "head_dim": wl.D, "global_seq": wl.S,
                   "cp": wl.cp, "local_seq": wl.local_S, "rank": 0, "steps_per_pass": wl.cp,
                   "flops_per_pass": ring_flops(wl.H, wl.local_S, wl.S, wl.D)},
        "roofline": h["roofline"],
        "step_ms_in_pass": round(h["step_ms"], 4),
        "steps_union_tflops": h["steps_union_tflops"],
    }
    extra = {}
    if not args.headline_only:
        q, kp, vp = h.pop("inputs")
        for name in [x for x in args.only.split(",") if x]:
            try:
                extra[name] = EXTRAS[name](args, torch, ca, workloads, gen, dev)
            except Exception as e:  # report, do not hide
                extra[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        line["workloads"] = extra
    if not args.no_cpu_baseline:
        q, kp, vp = h["inputs"] if "inputs" in h else (q, kp, vp)
        log("[bench] cpu baseline (fp64 oracle sample)")
        line["cpu_baseline"] = cpu_baseline(q, kp, vp, wl.D)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
