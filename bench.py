"""Benchmark of the context-parallel attention hot path on one MI355X.

Headline (``value``): causal striped ring attention at S = 128k (32 heads of 128, cp = 8,
token t on rank t mod 8, 16384 local tokens per rank). One step is every rank's ring
pass run one after another on this GPU: per rank 8 online-max steps under the per-step
causal mask of the striped layout, each merged by the LSE rule into the rank's running
partial as it finishes (ring_attn_step_fold), with the K/V hops into rotating receive
buffers on a copy stream. value = algorithmic TFLOP/s of the
step, 4*H*D*(S(S+1)/2) flops (only the visible query-key pairs count), inputs resident in
HBM when timing starts.

Also reported (``workloads``): the Wan2.2 share (10 heads, S = 32768 over cp = 8) in its
key-split, hop-carrying form; the 720p const-max ring (40 heads, local 9450) with the
bound and the merge; DCP decode over two interleaved paged shards (KV GB/s); the DCP
prefill chunk; the tiny fp32 ring; and the contiguous causal contrast of the headline
(same attention, contiguous shards: rank r does r + 1/2 chunks of work).

``roofline`` is measured live for the dominant kernel, the headline's INCL step kernel
(attn_step_bf16, causal_incl mask, 16384 x 16384 queries x keys, 32 heads): back-to-back
launches on one stream bracketed by HIP events on that stream. ``--roofline-only`` runs
just that loop, for a profiler run of the kernel alone (``--roofline-only KERNEL`` does the
same for the other workloads' kernels). Each workload reports the same for its own step
kernel.

``cpu_baseline`` times the fp64 oracle on a bounded sample of the headline's query rows
(random rank, head and row; all visible keys). The same leg compares bounded samples of
every workload's GPU outputs with the oracle and reports the errors as ``parity``: it is
the only part of this file that runs the oracle.

``clock_mhz`` per leg: the GPU's shader clock sampled through amdsmi while the leg's
timed loop runs, with the socket power of the same window (``socket_power_w``; null where
amdsmi cannot read them). The MFMA legs run at the board's power limit, so their clock is
whatever that power allows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu-baseline]
                       [--only wan22,constmax,decode,prefill,tiny,contrast,copy]
                       [--roofline-only [incl|strict|wan22|wan22pair|wan22split|constmax|online720|merge|bound|decode|copy]]

Warm-up: W untimed steps, then more until the warm-up has kept the GPU busy for at least
one second, so the clock has settled whatever W is (after a few tens of milliseconds of
load the clock was still falling and the same passes ran 9% slower).
"""

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
MIN_WARM_MS = 1000.0          # warm-up floor in GPU time

# HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch),
# scaled by the plain-copy calibration: the copy kernel moving 2 GiB in and 2 GiB out read
# FETCH_SIZE = 1048597 KiB and WRITE_SIZE = 2097152 KiB, so fetch x 2.0, write x 1.0
# (profiles/kv_copy__calibration.txt).
# Each entry holds for the kernel source whose sha256 prefix it names; after an edit of that
# source the figure no longer describes the kernel and traffic is reported as null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
TRAFFIC = {
    "attn_step_bf16/striped_causal_128k_incl_fold": {"source": "attn_bf16.hip", "sha256": "51a4a685faeba44f",
                                                     "fetch_kib": 609969.8, "write_kib": 265080.8},
    "attn_step_pair_bf16/wan22_cp8_online": {"source": "attn_bf16.hip", "sha256": "51a4a685faeba44f",
                                              "fetch_kib": 43172.3, "write_kib": 20645.1},
    "attn_step_bf16/wan22_cp8_online_keysplit": {"source": "attn_bf16.hip", "sha256": "51a4a685faeba44f",
                                                 "fetch_kib": 57600.9, "write_kib": 63000.0},
    "attn_step_bf16/wan22_720p_constmax": {"source": "attn_bf16.hip", "sha256": "51a4a685faeba44f",
                                           "fetch_kib": 332391.1, "write_kib": 190612.2},
    "dcp_decode/dcp_decode_gqa": {"source": "decode.hip", "sha256": "a324b829ca6b6ff4",
                                  "fetch_kib": 2778052.6 + 14932.25, "write_kib": 31631.8 + 1040.0},
    "lse_merge/wan22_720p_constmax": {"source": "merge.hip", "sha256": "c788302e3d8b9dc0",
                                      "fetch_kib": 779655.5, "write_kib": 190477.2},
    "const_max_bound/wan22_720p_constmax": {"source": "bound.hip", "sha256": "5c362a4869e5af73",
                                            "fetch_kib": 378047.6 + 47348.4, "write_kib": 160.0 + 2584.7},
}


def traffic(key):
    import hashlib
    t = TRAFFIC.get(key)
    if t is None:
        return None
    path = os.path.join(ROOT, "context_attention_lse_amd", "csrc", t["source"])
    with open(path, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != t["sha256"]:
            return None
    return round((t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ring_flops(H, Sq, Sk, D):
    return 4.0 * H * Sq * Sk * D


def causal_flops(H, D, S, strict=False):
    """4*H*D flops per visible pair of a causal S x S block (j <= i, or j < i if strict)."""
    return 4.0 * H * D * (S * (S - 1) / 2 if strict else S * (S + 1) / 2)


class ClockSampler:
    """The GPU's shader clock while a leg runs, from the power firmware's metrics table
    (amdsmi gpu_metrics, current_gfxclks: one reading per XCD, averaged here). The table is
    refreshed about once a second, so a reading counts only once it has changed after the
    leg started (it then describes the leg), and a short leg is repeated for ~1.3 s."""

    def __init__(self):
        self.handle, self.err = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) != 1:
                self.err = f"{len(handles)} GPUs visible to amdsmi; clock not attributed"
                return
            self.amdsmi, self.handle = amdsmi, handles[0]
            self.read()
        except Exception as e:   # report, do not fail the bench
            self.handle, self.err = None, repr(e)[:120]

    def read(self):
        """(shader clock in MHz, socket power in W or None)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        xs = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 65535]
        clk = sum(xs) / len(xs) if xs else float(m["current_gfxclk"])
        pw = None
        for key in ("current_socket_power", "average_socket_power"):
            v = m.get(key)
            if isinstance(v, (int, float)) and 0 < v < 65535:
                pw = float(v)
                break
        return clk, pw

    def __call__(self, fn):
        """Runs fn() while sampling every 5 ms; returns (fn's result, clock summary or None)."""
        if self.handle is None:
            return fn(), None
        samples, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    samples.append(self.read())
                except Exception:
                    pass
                time.sleep(0.005)

        th = threading.Thread(target=loop, daemon=True)
        th.start()
        try:
            res = fn()
        finally:
            stop.set()
            th.join()
        # readings before the first refresh inside the leg describe what ran before it
        fresh = [x for i, x in enumerate(samples) if any(y != samples[0] for y in samples[:i + 1])]
        if not fresh:
            return res, None
        clks = [c for c, _ in fresh]
        pws = [p for _, p in fresh if p is not None]
        return res, {"mean": round(sum(clks) / len(clks)), "min": round(min(clks)), "max": round(max(clks)),
                     "readings": len(set(fresh)),
                     "socket_power_w": round(sum(pws) / len(pws)) if pws else None}

    def measure(self, torch, fn, min_s=1.3):
        """Repeats fn (GPU work on the current stream) for at least min_s and returns the
        clock summary of that window."""
        def run():
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < min_s:
                fn()
                torch.cuda.synchronize()
        return self(run)[1]


def timed(torch, fn, reps, warm_calls=2, stream=None):
    """Mean ms per call of fn (launches on the current stream) over ``reps`` calls, after
    ``warm_calls`` calls and at least MIN_WARM_MS / 4 of untimed GPU time."""
    st = stream or torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, spent = 0, 0.0
    while done < warm_calls or spent < MIN_WARM_MS / 4:
        e0.record(st)
        fn()
        e1.record(st)
        e1.synchronize()
        spent += e0.elapsed_time(e1)
        done += 1
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def kernel_roofline(ms, flops, name, per_launch, key=None, note=None):
    ach = flops / (ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
         "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic(key) if key else None,
         "kernel": name, "per_launch": per_launch, "kernel_ms": round(ms, 4)}
    if note:
        r["note"] = note
    return r


def hbm_roofline(ms, nbytes, name, per_launch, key=None):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic(key) if key else None, "kernel": name,
            "per_launch": per_launch, "kernel_ms": round(ms, 4)}


# ------------------------------------------------------------------ headline: striped causal 128k

def headline(args, torch, ca, workloads, gen, dev, clock):
    wl = workloads.workload("striped_causal_128k")
    log(f"[bench] {wl.name}: generating inputs")
    t = gen.ring_inputs(wl, dev)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, "striped")
    vp = ca.ring.chunk_pool(t["v"], wl.cp, "striped")
    qs = [ca.ring.shard(t["q"], wl.cp, r, "striped").contiguous() for r in range(wl.cp)]
    n = wl.local_S
    out = {"wl": wl, "t": t}

    log("[bench] roofline: the INCL and STRICT step kernels alone")
    o = torch.empty((1, wl.H, n, wl.D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, wl.H, n), dtype=torch.float32, device=dev)
    reps = 30   # about 60 ms per figure: shorter windows caught clock transitions
    # in the pass, step 0 (the rank's own chunk) writes the running partial and every later
    # step folds its partial into it (ring_attn_step_fold): the roofline times that form
    incl = lambda: ca.ring_attn_step(qs[7], kp[7], vp[7], mask="causal_incl", out=o, lse=lse)  # noqa: E731
    incl_fold = lambda: ca.ring_attn_step(qs[7], kp[6], vp[6], mask="causal_incl", out=o, lse=lse,  # noqa: E731
                                          fold=True)
    k_incl = timed(torch, incl, reps)
    incl()
    k_fold = timed(torch, incl_fold, reps)
    clk_incl = clock.measure(torch, incl_fold)
    fl_incl = causal_flops(wl.H, wl.D, n)
    out["roofline"] = kernel_roofline(
        k_fold, fl_incl, "attn_step_bf16<0, 1, false> (ring_attn_step_fold, mask causal_incl)",
        f"{fl_incl / 1e12:.4f} TFLOP = 4*H*D*Sq*(Sq+1)/2 visible pairs, H=32 Sq=Sk=16384 D=128",
        key="attn_step_bf16/striped_causal_128k_incl_fold",
        note=f"mean of {reps} back-to-back launches on one stream: rank 7's queries against rank 6's chunk, "
             "folded into the running partial as the pass does")
    out["roofline"]["clock_mhz"] = clk_incl
    # rank 0's queries against rank 7's chunk: a STRICT step, folded
    incl()
    k_strict = timed(torch, lambda: ca.ring_attn_step(qs[0], kp[7], vp[7], mask="causal_strict", out=o, lse=lse,
                                                       fold=True), reps)
    del o, lse

    log("[bench] headline: every rank's ring pass")
    copy_stream = ca.streams.side_streams(2)[0]   # a stream whose work overlaps the calling stream's
    # one compute stream folding each step into the running partial (no final merge), hops on a
    # copy stream, replayed as a HIP graph per rank. Eagerly, two compute streams each folding
    # (2-way merge) ran ranks 0 + 7 in 31.18 ms against 31.29 for this form, about what the graph
    # replay gains; that form is not captured (RingPass.capture refuses it).
    rps = [ca.ring.RingPass(qs[r], kp, vp, r, layout="striped", causal=True, copy_stream=copy_stream, fold=True,
                            compute_streams=1) for r in range(wl.cp)]
    # each rank's pass replayed as a captured HIP graph (+0.3% over issuing it eagerly)
    graphs = [rp.capture() for rp in rps]

    def step():
        for g in graphs:
            g.replay()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, spent = 0, 0.0
    while done < args.warmup or spent < MIN_WARM_MS:
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        spent += e0.elapsed_time(e1)
        done += 1
    out["warmup_done"] = done

    def timed_steps():
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms, clk = clock(timed_steps)
    total = causal_flops(wl.H, wl.D, wl.S)
    # per-rank pass times (a separate set of passes, one event pair per rank)
    nrep = 3
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in rps]
          for _ in range(nrep)]
    for k in range(nrep):
        for r, rp in enumerate(rps):
            ev[k][r][0].record()
            rp.run()
            ev[k][r][1].record()
    torch.cuda.synchronize()
    per_rank = [sum(ev[k][r][0].elapsed_time(ev[k][r][1]) for k in range(nrep)) / nrep for r in range(wl.cp)]
    mean = sum(per_rank) / len(per_rank)
    # step s of rank r reads rank (r - s) mod cp's chunk: INCL when that rank is <= r, else STRICT.
    # Step 0 starts the running partial; steps 1.. fold into it.
    kinds = [((r - s) % wl.cp <= r, s >= 1) for r in range(wl.cp) for s in range(wl.cp)]
    n_incl = sum(1 for inc, fold in kinds if inc and not fold)
    n_fold_incl = sum(1 for inc, fold in kinds if inc and fold)
    n_strict = sum(1 for inc, fold in kinds if not inc)
    kernels_ms = n_incl * k_incl + n_fold_incl * k_fold + n_strict * k_strict
    out.update({
        "ms": ms, "tflops": total / (ms * 1e-3) / 1e12, "flops": total, "clock_mhz": clk,
        "per_rank_ms": [round(x, 3) for x in per_rank],
        "rank_balance_max_over_mean": round(max(per_rank) / mean, 4),
        "ring_parallel_tflops": round(total / (wl.cp * max(per_rank) * 1e-3) / 1e12, 2),
        "step_kernels": {"incl_ms": round(k_incl, 4), "incl_fold_ms": round(k_fold, 4),
                         "strict_fold_ms": round(k_strict, 4), "incl_steps": n_incl, "incl_fold_steps": n_fold_incl,
                         "strict_steps": n_strict,
                         "strict_tflops": round(causal_flops(wl.H, wl.D, n, True) / (k_strict * 1e-3) / 1e12, 2)},
        "exposed_ms": round(ms - kernels_ms, 3),
        "exposed_note": (f"step time minus the sum of its kernels timed alone ({n_incl} INCL steps starting the "
                         f"partial, {n_fold_incl} folded INCL and {n_strict} folded STRICT steps): the hop copies on "
                         "the copy stream and launch gaps that the steps did not hide"),
        "hop_bytes_per_step": int(2 * kp[0].numel() * kp.element_size() * (wl.cp - 1) * wl.cp),
    })
    # outputs kept for the parity check: rank, head, rows -> host copies taken in the cpu leg
    out["rps"] = rps
    out["qs"], out["kp"], out["vp"] = qs, kp, vp
    return out


# ------------------------------------------------------------------ workloads

def step_pairs(torch, ca, q, kp, vp, n_steps, o_shape, dev, two_chunks=False):
    """The Wan2.2 pass's step form without its hops and merge: unsplit steps over chunks
    0..n-1, step s on compute stream s % 2, so two launches are in flight as in the pass,
    each stream's steps after its first folding into its running partial. two_chunks: each
    launch takes two consecutive chunks (ring_attn_step_pair), n/2 launches.
    Returns fn() (launches on the current stream's work order) and the launch count."""
    cur = torch.cuda.current_stream()
    aux = ca.streams.side_streams(2, dev)[1]   # overlaps the calling stream (its own hardware queue)
    outs = [(torch.empty(o_shape, dtype=torch.float32, device=dev),
             torch.empty(o_shape[:-1], dtype=torch.float32, device=dev)) for _ in range(2)]

    def fn():
        aux.wait_stream(cur)
        for s in range(n_steps // 2 if two_chunks else n_steps):
            st = cur if s % 2 == 0 else aux
            with torch.cuda.stream(st):
                if two_chunks:
                    ca.ring_attn_step_pair(q, kp[2 * s], vp[2 * s], kp[2 * s + 1], vp[2 * s + 1], out=outs[s % 2][0],
                                           lse=outs[s % 2][1], fold=s >= 2)
                else:
                    ca.ring_attn_step(q, kp[s], vp[s], out=outs[s % 2][0], lse=outs[s % 2][1], fold=s >= 2)
        cur.wait_stream(aux)
    return fn, (n_steps // 2 if two_chunks else n_steps)


def run_wan22(args, torch, ca, workloads, gen, dev, clock):
    wl = workloads.workload("wan22_cp8_online")
    log(f"[bench] {wl.name}")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    # unsplit steps, two launches in flight on two compute streams (160 query tiles each: one
    # alone leaves 96 of 256 CUs idle, two fill them), each launch computing two consecutive
    # chunks (ring_attn_step_pair: each query tile's Q load, prologue, epilogue and fold paid
    # once per two chunks), carrying the hops of the chunks two launches ahead and folding
    # into its stream's running partial (a 2-way merge at the end). Key-split steps (each
    # alone fills the device) ran the pass 10% slower: their segments' partial stores and
    # combines cost more than the overlap gives.
    rp = ca.ring.RingPass(q, kp, vp, 0, layout=wl.layout, variant="online", split=False, compute_streams=2,
                          fused_hops=True, fold=True, pair_steps=True)
    # the pass replayed as one captured HIP graph (its launches and stream joins, with no
    # per-launch gaps; 0.8% faster than issuing it eagerly)
    graph = rp.capture()
    # windows of tens of milliseconds: a few-millisecond window caught clock transitions
    ms = timed(torch, graph.replay, max(100, args.steps), warm_calls=max(10, args.warmup))
    clk = clock.measure(torch, graph.replay)
    # the same pass with one chunk per launch, for comparison
    rp1 = ca.ring.RingPass(q, kp, vp, 0, layout=wl.layout, variant="online", split=False, compute_streams=2,
                           fused_hops=True, fold=True)
    graph1 = rp1.capture()
    ms1 = timed(torch, graph1.replay, max(100, args.steps), warm_calls=10)
    fl_step = ring_flops(wl.H, wl.local_S, wl.local_S, wl.D)
    fl = ring_flops(wl.H, wl.local_S, wl.S, wl.D)
    pairs, n = step_pairs(torch, ca, q, kp, vp, wl.cp, (1, wl.H, wl.local_S, wl.D), dev, two_chunks=True)
    p_ms = timed(torch, pairs, max(40, args.steps)) / n
    # the key-split form a single step uses (one launch at a time, filling the device)
    ws = ca.step_workspace(q, kp[0])
    o = torch.empty((1, wl.H, wl.local_S, wl.D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, wl.H, wl.local_S), dtype=torch.float32, device=dev)
    k_ms = timed(torch, lambda: ca.ring_attn_step(q, kp[0], vp[0], out=o, lse=lse, workspace=ws), 200)
    graph.replay()   # the parity check below reads this replay's output
    return {"workload": wl.name, "config": "B=1 H=10 D=128 S=32768 cp=8 local=4096 bf16, QK RMS-normed, rank 0",
            "ms_per_pass": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "clock_mhz": clk,
            "form": "unsplit launches of two steps each (two chunks a launch), two in flight on two compute "
                    "streams, hops carried by the launches, each stream folding into a running partial, 2-way LSE "
                    "merge; the pass replayed as one captured HIP graph",
            "one_chunk_per_launch": {"ms_per_pass": round(ms1, 4), "tflops": round(fl / (ms1 * 1e-3) / 1e12, 2),
                                     "note": "the same pass with one chunk per launch (8 launches)"},
            "roofline": kernel_roofline(p_ms, 2 * fl_step,
                                        "attn_step_pair_bf16<false> (ring_attn_step_pair, folding, two launches in "
                                        "flight)",
                                        f"{2 * fl_step / 1e9:.2f} GFLOP = 2 chunks x 4*H*Sq*Sk*D, H=10 Sq=Sk=4096 D=128",
                                        key="attn_step_pair_bf16/wan22_cp8_online",
                                        note="effective time per launch: the pass's 4 launches without hops or merge, "
                                             "alternating over two streams and folding, total / 4"),
            "keysplit_step": {"kernel_ms": round(k_ms, 4), "tflops": round(fl_step / (k_ms * 1e-3) / 1e12, 2),
                              "frac_bf16_peak": round(fl_step / (k_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "traffic": traffic("attn_step_bf16/wan22_cp8_online_keysplit"),
                              "note": "attn_step_bf16<0, 0, true>: the same step cut into 240 key ranges with a "
                                      "workspace (the form one step alone uses); mean of 200 back-to-back launches"},
            "_keep": {"wl": wl, "t": t, "out": rp.out, "lse": rp.lse}}


def run_constmax(args, torch, ca, workloads, gen, dev, clock):
    wl = workloads.workload("wan22_720p_constmax")
    log(f"[bench] {wl.name}")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout).contiguous()
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    fl = ring_flops(wl.H, wl.local_S, wl.S, wl.D)
    fl_step = ring_flops(wl.H, wl.local_S, wl.local_S, wl.D)
    res = {"workload": wl.name, "config": "B=1 H=40 D=128 S=75600 cp=8 local=9450 bf16, QK RMS-normed, rank 0"}
    reps = max(3, args.steps // 4)
    # const-max steps carry their hops; the online pass keeps the copy stream (its unsplit
    # steps on two streams lost 0.9% with carried hops)
    rp = ca.ring.RingPass(q, kp, vp, 0, variant="constmax", fused_hops=True)
    ms = timed(torch, rp.run, reps)
    clk = clock.measure(torch, rp.run)
    acc = rp.acc
    cm_step = lambda: ca.ring_attn_const_max_step(q, kp[1], vp[1], rp.c, acc, 0)  # noqa: E731
    k_ms = timed(torch, cm_step, 30)
    k_clk = clock.measure(torch, cm_step)
    res["constmax"] = {"ms_per_pass": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                       "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "clock_mhz": clk,
                       "roofline": kernel_roofline(
                           k_ms, fl_step, "attn_step_bf16<1, 0, false> (ring_attn_const_max_step, accumulate phase)",
                           f"{fl_step / 1e12:.4f} TFLOP = 4*H*Sq*Sk*D, H=40 Sq=Sk=9450 D=128",
                           key="attn_step_bf16/wan22_720p_constmax",
                           note="mean of 30 back-to-back launches on one stream")}
    res["constmax"]["roofline"]["clock_mhz"] = k_clk
    rp.run()
    keep = {"wl": wl, "t": t, "out": rp.out.clone(), "lse": rp.lse.clone()}
    # bound prologue: |k|^2 max over all 8 chunks + c for every query row (HBM-bound)
    ms_b = timed(torch, rp.prologue, 100)
    clk_b = clock.measure(torch, rp.prologue)
    nbytes = (kp.numel() + q.numel()) * kp.element_size() + q.shape[1] * wl.H * 4
    res["bound"] = {"ms": round(ms_b, 4), "bytes": nbytes, "GBps": round(nbytes / (ms_b * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(nbytes / (ms_b * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "clock_mhz": clk_b,
                    "roofline": hbm_roofline(ms_b, nbytes, "key_sqnorm_max_kernel + const_max_bound_kernel",
                                             "2*D bytes per key (8 chunks of 9450 x 40 heads) and per query row, "
                                             "+ 4 per c", "const_max_bound/wan22_720p_constmax")}
    del rp
    # sink-robust pass (theta 4): on these QK-normed keys no key qualifies, so this measures
    # what the sink prologue, the per-tile sink test and the sink merge cost
    rp = ca.ring.RingPass(q, kp, vp, 0, variant="constmax", sink_theta=4.0)
    ms_s = timed(torch, rp.run, max(2, reps // 2))
    res["constmax_sinks"] = {"ms_per_pass": round(ms_s, 4), "tflops": round(fl / (ms_s * 1e-3) / 1e12, 2),
                             "sinks_found": int(rp.sinks["sink_cnt"].sum().item())}
    del rp
    # two compute streams, each folding its steps into a running partial, a 2-way merge at the
    # end (12.61 ms against 12.70 for separate partials and an 8-way merge)
    rp = ca.ring.RingPass(q, kp, vp, 0, variant="online", fold=True, compute_streams=2)
    ms_o = timed(torch, rp.run, reps)
    o = torch.empty((1, wl.H, wl.local_S, wl.D), dtype=torch.float32, device=dev)
    lse = torch.empty((1, wl.H, wl.local_S), dtype=torch.float32, device=dev)
    k_on = timed(torch, lambda: ca.ring_attn_step(q, kp[1], vp[1], out=o, lse=lse), 30)
    res["online"] = {"ms_per_pass": round(ms_o, 4), "tflops": round(fl / (ms_o * 1e-3) / 1e12, 2),
                     "form": "unsplit steps on two compute streams, each folding into a running partial, 2-way "
                             "LSE merge; hops on a copy stream",
                     "step_kernel_ms": round(k_on, 4),
                     "step_tflops": round(fl_step / (k_on * 1e-3) / 1e12, 2),
                     "frac_bf16_peak_step": round(fl_step / (k_on * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del rp
    # the 8-way merge of the online partials (HBM-bound: 8 x 193.5 MB in, 195 MB out), on the
    # partials of a pass that keeps one per step
    rp = ca.ring.RingPass(q, kp, vp, 0, variant="online")
    rp.run()
    parts_o, parts_l = rp.o_parts[:wl.cp], rp.lse_parts[:wl.cp]
    merge = lambda: ca.lse_merge(parts_o, parts_l, out=rp.out, lse_out=rp.lse)  # noqa: E731
    ms_m = timed(torch, merge, 50)
    clk_m = clock.measure(torch, merge)
    nbytes = (parts_o.numel() + parts_l.numel()) * 4 + (rp.out.numel() + rp.lse.numel()) * 4
    res["merge"] = {"ms": round(ms_m, 4), "bytes": nbytes, "GBps": round(nbytes / (ms_m * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(nbytes / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "clock_mhz": clk_m,
                    "roofline": hbm_roofline(ms_m, nbytes, "lse_merge_kernel<128, false>",
                                             "n*rows*(D+1)*4 read + rows*(D+1)*4 written, n=8 rows=40*9450 D=128",
                                             "lse_merge/wan22_720p_constmax")}
    del rp
    res["_keep"] = keep
    return res


def run_decode(args, torch, ca, workloads, gen, dev, clock):
    wl = workloads.workload("dcp_decode_gqa")
    log(f"[bench] {wl.name}: building paged shards")
    d = gen.decode_inputs(wl, dev)
    shards = [ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], r, wl.shards,
                                       wl.interleave, wl.block_size, d["block_rand"]) for r in range(wl.shards)]
    run = ca.dcp.DcpDecode(d["q"], shards)
    steps = max(10, args.steps)
    kv_bytes = sum(sc.nbytes_kv for sc in shards)
    ms = timed(torch, run.run, steps)
    clk = clock.measure(torch, run.run)
    out, lse = run.run()
    keep = {"wl": wl, "d": d, "out": out.clone(), "lse": lse.clone(), "o_parts": run.o_parts.clone(),
            "lse_parts": run.lse_parts.clone()}
    shard_ms = [timed(torch, lambda sc=sc, r=r: ca.dcp_decode_partial(
        run.q, sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens, out=run.o_parts[r], lse=run.lse_parts[r],
        workspace=run.ws[r]), steps) for r, sc in enumerate(shards)]
    per_launch = [sc.nbytes_kv / (m * 1e-3) / 1e9 for sc, m in zip(shards, shard_ms)]
    ach = sum(per_launch) / len(per_launch)
    # the same step with a current token: the caches hold positions [0, N) of each sequence
    # and the new token at position N joins on its owner shard only (dcp_active_mask)
    prior = torch.tensor([int(n) for n in d["ctx"]], dtype=torch.int32, device=dev)
    k_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 21, dev, torch.bfloat16)
    v_cur = gen.normal((wl.B, wl.Hkv, wl.D), 1000 * wl.seed + 22, dev, torch.bfloat16)
    ms_active = timed(torch, lambda: run.run_active(prior, k_cur, v_cur, wl.interleave), steps)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    return {"workload": wl.name, "config": "B=32 Hq=64 Hkv=8 D=128 bf16, ctx U[32k,128k], block 16, 2 interleaved shards",
            "kv_bytes": kv_bytes, "ms_per_step": round(ms, 4), "kv_GBps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "clock_mhz": clk,
            "with_current_token": {"ms_per_step": round(ms_active, 4),
                                   "kv_GBps": round(kv_bytes / (ms_active * 1e-3) / 1e9, 1),
                                   "note": "N resident tokens on their shards plus a new token at position N, "
                                           "attended on its owner shard only"},
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic("dcp_decode/dcp_decode_gqa"),
                         "kernel": "dcp_decode_split_kernel + combine (dcp_decode_partial)",
                         "per_launch": "one shard's resident K+V bytes = local tokens * Hkv * D * 2 * 2",
                         "kernel_ms": [round(m, 4) for m in shard_ms]},
            "_keep": keep}


def run_prefill(args, torch, ca, workloads, gen, dev, clock):
    """DCP prefill of one chunk (segmented attention on every rank + the LSE merge):
    S = 8192 new tokens after 65536 prior ones, 32 query heads over 8 KV heads, D = 128,
    DCP = 2 ranks interleaving blocks of 16, bf16; synthetic N(0, 1) inputs."""
    import numpy as np
    S, P, Hq, Hkv, D, W, I = 8192, 65536, 32, 8, 128, 2, 16
    log("[bench] dcp prefill")
    q = gen.normal((1, S, Hq, D), 901, dev, torch.bfloat16)
    k_all = gen.normal((P + S, Hkv, D), 902, dev, torch.bfloat16)
    v_all = gen.normal((P + S, Hkv, D), 903, dev, torch.bfloat16)
    caches = [ca.dcp.build_shard_cache(k_all, v_all, np.array([0, P]), np.array([P]), r, W, I, 16) for r in range(W)]
    run = ca.dcp.DcpPrefill(q, k_all[P:].unsqueeze(0), v_all[P:].unsqueeze(0), caches, P, I)
    del k_all, v_all
    ms = timed(torch, run.run, max(3, args.steps // 4))
    clk = clock.measure(torch, run.run)
    flops = 4.0 * Hq * D * (S * P + S * (S + 1) / 2)
    return {"workload": "dcp_prefill_chunk", "config": f"S={S} after {P} prior, Hq={Hq} Hkv={Hkv} D={D}, DCP={W} "
            f"interleave {I}, bf16, both ranks + merge", "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "clock_mhz": clk}


def run_tiny(args, torch, ca, workloads, gen, dev, clock):
    wl = workloads.workload("tiny_ring_fp32")
    t = gen.ring_inputs(wl, dev)
    q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout).contiguous()
    kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
    vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
    res = {"workload": wl.name, "config": "B=1 H=2 D=64 S=512 cp=4 fp32, rank 0"}
    keep = {"wl": wl, "t": t}
    for variant in ("online", "constmax"):
        rp = ca.ring.RingPass(q, kp, vp, 0, variant=variant)
        res[f"{variant}_ms_per_pass"] = round(timed(torch, rp.run, 10), 4)
        o, l = rp.run()
        keep[variant] = (o.clone(), l.clone())
    res["_keep"] = keep
    return res


def run_contrast(args, torch, ca, workloads, gen, dev, clock, t=None):
    """Contiguous causal ring on the headline's inputs: rank r sees r full chunks and its own
    triangle, so the ranks' work differs (Sharding the Input, Striped Attention)."""
    wl = workloads.workload("contiguous_causal_128k")
    log(f"[bench] {wl.name}")
    if t is None:
        t = gen.ring_inputs(wl, dev)
    kp = ca.ring.chunk_pool(t["k"], wl.cp, "contiguous")
    vp = ca.ring.chunk_pool(t["v"], wl.cp, "contiguous")
    copy_stream = ca.streams.side_streams(2)[0]
    per_rank = []
    for r in range(wl.cp):
        q = ca.ring.shard(t["q"], wl.cp, r, "contiguous").contiguous()
        rp = ca.ring.RingPass(q, kp, vp, r, layout="contiguous", causal=True, copy_stream=copy_stream)
        per_rank.append(timed(torch, rp.run, 2, warm_calls=1))
        del rp, q
    total = causal_flops(wl.H, wl.D, wl.S)
    mean = sum(per_rank) / len(per_rank)
    return {"workload": wl.name, "config": "B=1 H=32 D=128 S=131072 cp=8 contiguous causal bf16, all 8 ranks",
            "ms_all_ranks": round(sum(per_rank), 3), "tflops": round(total / (sum(per_rank) * 1e-3) / 1e12, 2),
            "per_rank_ms": [round(x, 3) for x in per_rank],
            "rank_balance_max_over_mean": round(max(per_rank) / mean, 4),
            "ring_parallel_tflops": round(total / (wl.cp * max(per_rank) * 1e-3) / 1e12, 2),
            "note": "ring_parallel_tflops: the rate if the ranks ran at once on cp GPUs and the slowest set the "
                    "pace; striped sharding (the headline) balances the ranks, contiguous does not"}


def run_copy(args, torch, ca, workloads, gen, dev, clock):
    n = 1 << 29                      # 2**29 bf16 = 1 GiB per tensor
    src_k = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    src_v = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    dst_k = torch.empty_like(src_k)
    dst_v = torch.empty_like(src_v)
    ms = timed(torch, lambda: ca.kv_chunk_copy(dst_k, dst_v, src_k, src_v), 3)
    nbytes = 4 * n * 2                # read 2 GiB + write 2 GiB per call
    return {"workload": "device copy 2 x 1 GiB", "ms_per_call": round(ms, 4),
            "bytes_read_per_call": 2 * n * 2, "bytes_written_per_call": 2 * n * 2,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


EXTRAS = {"wan22": run_wan22, "constmax": run_constmax, "decode": run_decode, "prefill": run_prefill,
          "tiny": run_tiny, "contrast": run_contrast, "copy": run_copy}


# ------------------------------------------------------------------ the oracle leg

def cpu_baseline_leg(h, kept, budget_s=12.0):
    """The only use of the oracle in this file. (1) cpu_baseline: the fp64 oracle on random
    query rows of the headline (random rank, head and row; each row against every key it
    may see, under the striped causal mask), until about budget_s of CPU time, scaled to the
    headline's unit (algorithmic TFLOP/s of the sampled rows). The same rows' GPU outputs
    are compared with it. (2) parity: bounded samples of the other workloads' GPU outputs
    against the oracle."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    parity = {}

    def err(o_gpu, l_gpu, ro, rl):
        o_gpu = o_gpu.detach().double().cpu().numpy()
        l_gpu = l_gpu.detach().double().cpu().numpy()
        fin = np.isfinite(rl)
        if not np.array_equal(np.isfinite(l_gpu), fin):
            return float("inf"), float("inf")
        eo = float(np.abs(o_gpu - ro).max()) if ro.size else 0.0
        el = float(np.abs(l_gpu[fin] - rl[fin]).max()) if fin.any() else 0.0
        return eo, el

    def entry(eo, el, rows, what, secs, scale_up, how):
        # secs: oracle wall time on the sample; scale_up: the whole workload's result over the
        # sample's (by rows, visible pairs or tokens, as `how` says)
        return {"max_abs_dO": eo, "max_abs_dLSE": el, "rows_checked": rows, "what": what,
                "pass": bool(eo <= 2e-2 and el <= 1e-3), "oracle_s": round(secs, 3),
                "oracle_full_s": round(secs * scale_up, 1),
                "oracle_full_how": "measured" if scale_up == 1 else f"extrapolated from the sample {how}"}

    def timed_oracle(fn, *a):
        t0 = time.perf_counter()
        r = fn(*a)
        return r, time.perf_counter() - t0

    # (1) headline rows
    wl, t = h["wl"], h["t"]
    S, n, cp, D = wl.S, wl.local_S, wl.cp, wl.D
    scale = oracle.default_scale(D)
    rng = np.random.default_rng(5)
    rows_done, flops, t_total, eo, el = 0, 0.0, 0.0, 0.0, 0.0
    k_cache, batch = {}, 16
    while t_total < budget_s and rows_done < 4096:
        r = int(rng.integers(cp))
        hh = int(rng.integers(wl.H))
        rows = np.sort(rng.choice(n, size=batch, replace=False))
        if hh not in k_cache:
            k_cache.clear()
            k_cache[hh] = (t["k"][0, :, hh].cpu(), t["v"][0, :, hh].cpu())
        kh, vh = k_cache[hh]
        tok = oracle.striped_tokens(S, cp, r)[rows]
        q_rows = t["q"][0, tok, hh].cpu()
        t0 = time.perf_counter()
        ro, rl = oracle.attention(q_rows, kh, vh, scale, oracle.causal_allowed(tok, np.arange(S)))
        t_total += time.perf_counter() - t0
        rows_done += batch
        flops += 4.0 * D * float((tok + 1).sum())
        rp = h["rps"][r]
        e = err(rp.out[0, hh, torch.from_numpy(rows).to(rp.out.device)], rp.lse[0, hh, torch.from_numpy(rows).to(
            rp.out.device)], ro, rl)
        eo, el = max(eo, e[0]), max(el, e[1])
    cpu = {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows_done} random query rows of the headline (random rank and head), each against every key "
                     f"it may see under the striped causal mask (fp64 numpy oracle, {t_total:.1f} s; the oracle "
                     f"scores every key and masks, so it does twice the algorithmic work counted)"}
    parity[wl.name] = entry(eo, el, rows_done, "random rows of random ranks and heads, all visible keys", t_total,
                            wl.H * S / rows_done, "by rows (every rank and head; each row costs the oracle all S keys)")

    # (2) other workloads
    if "wan22" in kept:
        k = kept["wan22"]
        w, tt = k["wl"], k["t"]
        tok = oracle.contiguous_tokens(w.S, w.cp, 0)
        eo = el = secs = 0.0
        for hh in (0, w.H - 1):
            (ro, rl), dt = timed_oracle(oracle.attention, tt["q"][0, tok, hh].cpu(), tt["k"][0, :, hh].cpu(),
                                        tt["v"][0, :, hh].cpu(), oracle.default_scale(w.D))
            secs += dt
            e = err(k["out"][0, hh], k["lse"][0, hh], ro, rl)
            eo, el = max(eo, e[0]), max(el, e[1])
        parity[w.name] = entry(eo, el, 2 * w.local_S, "every row of heads 0 and 9 of rank 0's pass", secs, w.H / 2,
                               "by rows (rank 0's pass, all heads)")
    if "constmax" in kept:
        k = kept["constmax"]
        w, tt = k["wl"], k["t"]
        tok = oracle.contiguous_tokens(w.S, w.cp, 0)
        eo = el = secs = 0.0
        rows_n = 0
        for hh in (0, 13, 26, w.H - 1):
            rows = np.unique(np.concatenate([np.random.default_rng(hh).choice(w.local_S, 96, replace=False),
                                             np.arange(w.local_S - 106, w.local_S, 8)]))
            (ro, rl), dt = timed_oracle(oracle.attention, tt["q"][0, tok[rows], hh].cpu(), tt["k"][0, :, hh].cpu(),
                                        tt["v"][0, :, hh].cpu(), oracle.default_scale(w.D))
            secs += dt
            ix = torch.from_numpy(rows).to(k["out"].device)
            e = err(k["out"][0, hh, ix], k["lse"][0, hh, ix], ro, rl)
            eo, el = max(eo, e[0]), max(el, e[1])
            rows_n += len(rows)
        parity[w.name + "/constmax"] = entry(eo, el, rows_n, "random rows and the ragged tail of 4 heads", secs,
                                             w.H * w.local_S / rows_n, "by rows (rank 0's pass, all heads)")
    if "decode" in kept:
        k = kept["decode"]
        w, d = k["wl"], k["d"]
        G = w.Hq // w.Hkv
        ctx = d["ctx"]
        seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 7, 19})
        eo = el = secs = 0.0
        for b in seqs:
            s0, s1 = int(d["offsets"][b]), int(d["offsets"][b + 1])
            for hk in range(w.Hkv):
                hs = slice(hk * G, (hk + 1) * G)
                (ro, rl), dt = timed_oracle(oracle.attention, d["q"][b, hs].cpu(), d["k_seq"][s0:s1, hk].cpu(),
                                            d["v_seq"][s0:s1, hk].cpu(), oracle.default_scale(w.D))
                secs += dt
                e = err(k["out"][b, hs], k["lse"][b, hs], ro, rl)
                eo, el = max(eo, e[0]), max(el, e[1])
        parity[w.name] = entry(eo, el, len(seqs) * w.Hq, f"sequences {seqs}, every query head, merged over both shards",
                               secs, float(np.sum(ctx)) / float(np.sum(ctx[seqs])), "by context tokens")
    if "tiny" in kept:
        k = kept["tiny"]
        w, tt = k["wl"], k["t"]
        tok = oracle.contiguous_tokens(w.S, w.cp, 0)
        (ro, rl), secs = timed_oracle(oracle.attention_heads, tt["q"][:, tok].cpu(), tt["k"].cpu(), tt["v"].cpu(),
                                      oracle.default_scale(w.D))
        for variant in ("online", "constmax"):
            o, l = k[variant]
            e = err(o, l, ro, rl)
            parity[f"{w.name}/{variant}"] = {"max_abs_dO": e[0], "max_abs_dLSE": e[1], "rows_checked": w.local_S * w.H,
                                             "what": "every row (fp32 path; bar 1e-4 on both)",
                                             "pass": bool(e[0] <= 1e-4 and e[1] <= 1e-4), "oracle_s": round(secs, 3),
                                             "oracle_full_s": round(secs, 3), "oracle_full_how": "measured"}
    return cpu, parity


def profile_kernel(name, torch, ca, workloads, gen, dev, reps=10):
    """Back-to-back launches of one kernel on one stream with a workload's inputs (for a
    profiler run of that kernel alone); prints its roofline figures. Kernels:
    incl, strict  the headline's step kernel under the INCL / STRICT mask (32 heads, 16384^2),
                  folding into a running partial as the pass does
    wan22         the Wan2.2 share's unsplit step as its pass runs it: 8 launches (chunks 0..7)
                  alternating over two streams, two in flight, each stream's later steps
                  folding (10 heads, 4096^2); the figures are per launch (total / 8)
    wan22pair     the Wan2.2 pass's launches of two chunks each (ring_attn_step_pair), 4 launches
                  alternating over two streams, folding; the figures are per launch (total / 4)
    wan22split    the same step cut into key ranges (the form one step alone uses)
    constmax      the 720p const-max step, accumulate phase (40 heads, 9450^2)
    online720     the 720p online step
    merge         the 720p 8-way LSE merge (8 x 40 x 9450 rows of 128)
    bound         the 720p bound prologue (key norms over all 8 chunks, then c per query row)
    decode        one DCP decode shard of the decode workload (both kernels of the call)
    copy          the plain K/V copy of 2 x 1 GiB (calibrates the HBM byte counters)"""
    import math
    if name in ("incl", "strict"):
        wl = workloads.workload("striped_causal_128k")
        t = gen.ring_inputs(wl, dev)
        kp = ca.ring.chunk_pool(t["k"], wl.cp, "striped")
        vp = ca.ring.chunk_pool(t["v"], wl.cp, "striped")
        r, src = (7, 7) if name == "incl" else (0, 7)
        q = ca.ring.shard(t["q"], wl.cp, r, "striped").contiguous()
        del t
        n = wl.local_S
        o = torch.empty((1, wl.H, n, wl.D), dtype=torch.float32, device=dev)
        lse = torch.empty((1, wl.H, n), dtype=torch.float32, device=dev)
        mask = "causal_incl" if name == "incl" else "causal_strict"
        # the pass's form: the step's partial folded into the running one
        ca.ring_attn_step(q, kp[r], vp[r], mask="causal_incl", out=o, lse=lse)
        src = 6 if name == "incl" else 7
        fn = lambda: ca.ring_attn_step(q, kp[src], vp[src], mask=mask, out=o, lse=lse, fold=True)  # noqa: E731
        work = causal_flops(wl.H, wl.D, n, strict=(name == "strict"))
        unit, per = "flop", f"4*H*D*visible pairs, H=32 Sq=Sk=16384 D=128, mask {mask}"
    elif name in ("wan22", "wan22split", "wan22pair"):
        wl = workloads.workload("wan22_cp8_online")
        t = gen.ring_inputs(wl, dev)
        q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout)
        kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
        vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
        work = ring_flops(wl.H, wl.local_S, wl.local_S, wl.D)
        if name == "wan22":
            fn, launches = step_pairs(torch, ca, q, kp, vp, wl.cp, (1, wl.H, wl.local_S, wl.D), dev)
            unit, per = "flop", "4*H*Sq*Sk*D, H=10 Sq=Sk=4096 D=128, unsplit, two launches in flight"
            reps = 5
        elif name == "wan22pair":
            fn, launches = step_pairs(torch, ca, q, kp, vp, wl.cp, (1, wl.H, wl.local_S, wl.D), dev, two_chunks=True)
            work *= 2
            unit, per = "flop", "2 chunks x 4*H*Sq*Sk*D, H=10 Sq=Sk=4096 D=128, two launches in flight"
            reps = 5
        else:
            ws = ca.step_workspace(q, kp[0])
            o = torch.empty((1, wl.H, wl.local_S, wl.D), dtype=torch.float32, device=dev)
            lse = torch.empty((1, wl.H, wl.local_S), dtype=torch.float32, device=dev)
            fn = lambda: ca.ring_attn_step(q, kp[0], vp[0], out=o, lse=lse, workspace=ws)  # noqa: E731
            unit, per = "flop", "4*H*Sq*Sk*D, H=10 Sq=Sk=4096 D=128, key-split"
            reps = 30
    elif name in ("constmax", "online720", "merge", "bound"):
        wl = workloads.workload("wan22_720p_constmax")
        t = gen.ring_inputs(wl, dev)
        q = ca.ring.shard(t["q"], wl.cp, 0, wl.layout).contiguous()
        kp = ca.ring.chunk_pool(t["k"], wl.cp, wl.layout)
        vp = ca.ring.chunk_pool(t["v"], wl.cp, wl.layout)
        del t
        n, H, D = wl.local_S, wl.H, wl.D
        if name == "constmax":
            rp = ca.ring.RingPass(q, kp, vp, 0, variant="constmax")
            rp.run()
            fn = lambda: ca.ring_attn_const_max_step(q, kp[1], vp[1], rp.c, rp.acc, 0)  # noqa: E731
            work, unit, per = ring_flops(H, n, n, D), "flop", "4*H*Sq*Sk*D, H=40 Sq=Sk=9450 D=128"
        elif name == "online720":
            o = torch.empty((1, H, n, D), dtype=torch.float32, device=dev)
            lse = torch.empty((1, H, n), dtype=torch.float32, device=dev)
            fn = lambda: ca.ring_attn_step(q, kp[1], vp[1], out=o, lse=lse)  # noqa: E731
            work, unit, per = ring_flops(H, n, n, D), "flop", "4*H*Sq*Sk*D, H=40 Sq=Sk=9450 D=128"
        elif name == "merge":
            rp = ca.ring.RingPass(q, kp, vp, 0, variant="online")
            rp.run()
            po, pl = rp.o_parts[:wl.cp], rp.lse_parts[:wl.cp]
            fn = lambda: ca.lse_merge(po, pl, out=rp.out, lse_out=rp.lse)  # noqa: E731
            work = (po.numel() + pl.numel()) * 4 + (rp.out.numel() + rp.lse.numel()) * 4
            unit, per = "byte", "n*rows*(D+1)*4 read + rows*(D+1)*4 written, n=8 rows=40*9450 D=128"
            reps = 30
        else:
            rp = ca.ring.RingPass(q, kp, vp, 0, variant="constmax")
            fn = rp.prologue
            work = (kp.numel() + q.numel()) * kp.element_size() + n * H * 4
            unit, per = "byte", "2*D bytes per key (8 chunks of 9450 x 40 heads) and per query row, + 4 per c"
            reps = 30
    elif name == "decode":
        wl = workloads.workload("dcp_decode_gqa")
        d = gen.decode_inputs(wl, dev)
        sc = ca.dcp.build_shard_cache(d["k_seq"], d["v_seq"], d["offsets"], d["ctx"], 0, wl.shards, wl.interleave,
                                      wl.block_size, d["block_rand"])
        del d["k_seq"], d["v_seq"]
        run = ca.dcp.DcpDecode(d["q"], [sc])
        fn = lambda: ca.dcp_decode_partial(run.q, sc.k_pool, sc.v_pool, sc.block_table, sc.local_lens,  # noqa: E731
                                           out=run.o_parts[0], lse=run.lse_parts[0], workspace=run.ws[0])
        work, unit, per = sc.nbytes_kv, "byte", "shard 0's resident K+V bytes = local tokens * Hkv * D * 2 * 2"
        reps = 20
    elif name == "copy":
        # the calibration copy of the HBM byte counters: 1 GiB of K and 1 GiB of V per call
        nel = 1 << 29
        src_k = torch.zeros(nel, dtype=torch.bfloat16, device=dev)
        src_v = torch.zeros(nel, dtype=torch.bfloat16, device=dev)
        dst_k, dst_v = torch.empty_like(src_k), torch.empty_like(src_v)
        fn = lambda: ca.kv_chunk_copy(dst_k, dst_v, src_k, src_v)  # noqa: E731
        work, unit, per = 4 * nel * 2, "byte", "2 GiB read + 2 GiB written"
        reps = 3
    else:
        raise SystemExit(f"unknown kernel {name!r}")
    ms = timed(torch, fn, reps)
    if name in ("wan22", "wan22pair"):
        ms /= launches
    rate = work / (ms * 1e-3)
    if unit == "flop":
        res = {"bound": "mfma", "achieved": round(rate / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
               "frac": round(rate / 1e12 / PEAK_BF16_TFLOPS, 4)}
    else:
        res = {"bound": "hbm", "achieved": round(rate / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": round(rate / 1e9 / PEAK_HBM_GBS, 4)}
    res.update({"kernel_ms": round(ms, 4), "per_launch": f"{work:.6g} {unit}s = {per}", "launches_timed": reps})
    assert math.isfinite(ms)
    print(json.dumps({"kernel": name, "roofline": res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--roofline-only", nargs="?", const="incl", default=None,
                    choices=["incl", "strict", "wan22", "wan22pair", "wan22split", "constmax", "online720", "merge",
                             "bound",
                             "decode", "copy"],
                    help="time one kernel alone, back to back (for profiling it); default: the headline's "
                         "INCL step kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="wan22,constmax,decode,prefill,tiny,contrast",
                    help="comma-separated extra workloads to run after the headline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ring's ranks run one after another on that device, so "
              "--gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import context_attention_lse_amd as ca
    import workloads
    from workloads import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ca._lib.load()
    clock = ClockSampler()

    if args.roofline_only:
        profile_kernel(args.roofline_only, torch, ca, workloads, gen, dev)
        return
    h = headline(args, torch, ca, workloads, gen, dev, clock)
    wl = h["wl"]
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
        "data": "synthetic (seeded torch.randn N(0,1) Q, K, V)",
        "config": {"workload": wl.name, "B": wl.B, "heads": wl.H, "head_dim": wl.D, "global_seq": wl.S,
                   "cp": wl.cp, "local_seq": wl.local_S, "layout": "striped", "causal": True,
                   "ranks_per_step": wl.cp, "ring_steps_per_rank": wl.cp, "flops_per_step": h["flops"]},
        "step": "every rank's ring pass (8 steps, each folded by the LSE rule into the running partial; hops on a "
                "copy stream), ranks one after another, each pass replayed as a captured HIP graph",
        "frac_bf16_peak": round(h["tflops"] / PEAK_BF16_TFLOPS, 4),
        "roofline": h["roofline"],
        "clock_mhz": h["clock_mhz"],
        "warmup_steps_done": h["warmup_done"],
        "per_rank_ms": h["per_rank_ms"],
        "rank_balance_max_over_mean": h["rank_balance_max_over_mean"],
        "ring_parallel_tflops": h["ring_parallel_tflops"],
        "step_kernels": h["step_kernels"],
        "exposed_ms": h["exposed_ms"],
        "exposed_note": h["exposed_note"],
        "hop_bytes_per_step": h["hop_bytes_per_step"],
    }
    if clock.err:
        line["clock_error"] = clock.err
    extra, kept = {}, {}
    if not args.headline_only:
        for name in [x for x in args.only.split(",") if x]:
            try:
                if name == "contrast":
                    extra[name] = run_contrast(args, torch, ca, workloads, gen, dev, clock, t=h["t"])
                else:
                    extra[name] = EXTRAS[name](args, torch, ca, workloads, gen, dev, clock)
                if "_keep" in extra[name]:
                    kept[name] = extra[name].pop("_keep")
            except Exception as e:  # report, do not hide
                extra[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        line["workloads"] = extra
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline and parity samples (fp64 oracle)")
        line["cpu_baseline"], line["parity"] = cpu_baseline_leg(h, kept)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
