"""One rank's ring attention on one GPU: resident queries, K/V chunks delivered step by
step, partials merged by LSE (or folded by the const-max rule).

The ring schedule follows "Kernel reference: ring_attention_const_max_fwd" (Overview
figure and Implementation, "The ring loop"): step 0 uses the rank's own K/V, step s
uses the chunk of rank r - s (mod cp); the hop for step s + depth is launched before
step s computes, into one of depth + 1 rotating buffers. On one GPU the other ranks'
chunks sit in a pool in HBM and each hop is a device copy (kv_chunk_copy) on a copy
stream, ordered against the compute stream by events.

Striped sharding and its causal mask follow "Sharding the Input" (Striped Attention):
token t lives on rank t mod cp at local index t div cp, so key (j, rank r') is visible
to query (i, rank r) iff j*cp + r' <= i*cp + r, i.e. j <= i when r' <= r and j < i
otherwise: one of two triangular masks per step.

This module only orders library calls; every byte of arithmetic runs in libctxattn.
"""

import torch

from . import api
from .streams import side_streams

LAYOUTS = ("contiguous", "striped")


def check_divisible(S: int, cp: int) -> None:
    """Sequence length must divide by the ring size (context-parallelism page,
    sequence sharding); the error names both numbers."""
    if cp <= 0:
        raise ValueError(f"cp must be positive, got {cp}")
    if S % cp:
        raise ValueError(f"Sequence length {S} is not divisible by cp_size {cp}.")


def ring_source_rank(rank: int, step: int, cp: int) -> int:
    """Rank whose K/V chunk rank ``rank`` holds at ring step ``step``."""
    return (rank - step) % cp


def shard(x: torch.Tensor, cp: int, rank: int, layout: str) -> torch.Tensor:
    """Rank ``rank``'s tokens of a [B, S, H, D] tensor as a (possibly strided) view."""
    check_divisible(x.shape[1], cp)
    if layout == "contiguous":
        n = x.shape[1] // cp
        return x[:, rank * n:(rank + 1) * n]
    if layout == "striped":
        return x[:, rank::cp]
    raise ValueError(f"unknown layout {layout!r}")


def chunk_pool(x: torch.Tensor, cp: int, layout: str) -> torch.Tensor:
    """Every rank's shard, each contiguous: [cp, B, S/cp, H, D] (the peers' HBM)."""
    return torch.stack([shard(x, cp, r, layout).contiguous() for r in range(cp)], 0)


def step_mask(layout: str, causal: bool, query_rank: int, source_rank: int):
    """Mask of one step, or None when causality hides the whole chunk."""
    if not causal:
        return "none"
    if layout == "striped":
        return "causal_incl" if source_rank <= query_rank else "causal_strict"
    # contiguous: earlier chunks fully visible, own chunk triangular, later chunks hidden
    if source_rank < query_rank:
        return "none"
    if source_rank == query_rank:
        return "causal_incl"
    return None


class RingPass:
    """One rank's share of ring attention: q resident, cp chunks arriving one per step.

    variant "online": every step emits a partial (o_s, lse_s) with ring_attn_step and
                      the partials are merged once with lse_merge; with fold=True each
                      step instead merges its partial in place into its compute stream's
                      running partial (ring_attn_step_fold), and the streams' running
                      partials (one or two) are merged at the end;
    variant "constmax" with sink_theta: keys whose norm exceeds sink_theta x the mean key
                      norm (at most sink_cap per head) leave the bound and the fold, and are
                      attended exactly in a second partial merged by LSE;
    variant "constmax": the bound is built from every chunk's key norms (the ring's
                      all_reduce(max) becomes a max-fold), then every step adds into one
                      fp32 accumulator and the last step normalises.

    split=True gives the steps a key-split workspace where the library would split (query
    tiles too few to fill the device), so each step's grid fills it; such steps run on one
    compute stream by default. Otherwise steps keep one workgroup per query tile and online
    steps alternate two compute streams, so a step can fill the CUs the previous one leaves
    idle as it drains. compute_streams overrides either default. The copy stream and the
    second compute stream come from streams.side_streams (each checked to overlap the calling
    stream) unless copy_stream is given. On the Wan2.2 share (160 query tiles of 256 rows per
    step) the fastest pass is unsplit launches of two chunks each (pair_steps, below) on two
    streams with fused hops, each stream folding (0.652 ms replayed as a graph, against 0.671
    with one chunk a launch); key-split steps on two streams, also carrying the hops, took
    0.806 ms against 0.731 ms for unsplit ones when the two were last compared (before the
    folding).

    fused_hops=True (no sinks): each step call carries the hop of the chunk two steps ahead
    (ring_attn_step_hop, or ring_attn_step_fold_hop when folding), on the CUs the step leaves
    free when there are any, instead of a copy stream. A step fills every CU's register file,
    so a copy kernel on its own stream runs only between steps; carried by the step it costs
    nothing there. On the Wan2.2 share (240 ranges, 16 CUs free) the pass went from 806 to
    779 us. With fold as well, each compute stream folds its steps into one running partial
    and the pass ends in a 2-way merge instead of an 8-way one (Wan2.2, unsplit steps two in
    flight: 695 -> 687 us).

    pair_steps=True (online, non-causal, fold and fused_hops, bf16 D = 128, chunk length a
    multiple of 32): once two chunks have arrived, one launch computes both steps
    (ring_attn_step_pair), so each query tile's fixed work (Q load, copy prologue, epilogue,
    fold) is paid once per two chunks. Launches alternate the two compute streams as single
    steps do; launch i carries the hops of chunks 2i + 4 and 2i + 5 and every received chunk
    keeps a buffer of its own (cp - 1 of them).
    """

    def __init__(self, q, k_pool, v_pool, rank, *, layout="contiguous", causal=False, variant="online",
                 scale=None, prefetch_depth=2, out_dtype=torch.float32, copy_stream=None,
                 compute_streams=None, split=False, sink_theta=None, sink_cap=32, fold=False, fused_hops=False,
                 pair_steps=False):
        if variant not in ("online", "constmax"):
            raise ValueError(f"unknown variant {variant!r}")
        if fold and variant != "online":
            raise ValueError("fold applies to the online variant")
        if variant == "constmax" and causal:
            raise ValueError("the const-max method is non-causal")
        if layout not in LAYOUTS:
            raise ValueError(f"unknown layout {layout!r}")
        self.cp = k_pool.shape[0]
        if not (0 <= rank < self.cp):
            raise ValueError(f"rank {rank} outside ring of {self.cp}")
        self.q, self.k_pool, self.v_pool = q, k_pool, v_pool
        self.rank, self.layout, self.causal, self.variant = rank, layout, causal, variant
        self.scale = scale
        self.out_dtype = out_dtype
        self.depth = max(1, min(int(prefetch_depth), max(1, self.cp - 1)))
        self.nbuf = self.depth + 1
        # fused hops: step s carries the hop of chunk s + 2 (ring_attn_step_hop). Its buffer was
        # last read by step s - 2, which ran before it on the same compute stream; four
        # buffers keep that true with two compute streams.
        self.fused_hops = bool(fused_hops)
        if self.fused_hops:
            if sink_theta is not None:
                raise ValueError("fused hops do not combine with sinks")
            self.depth, self.nbuf = 2, 4
        B, Sq, H, D = q.shape
        self.pair_steps = bool(pair_steps)
        if self.pair_steps:
            if variant != "online" or causal or not fold or not self.fused_hops or split:
                raise ValueError("pair_steps: online, non-causal, with fold=True and fused_hops=True, no split")
            if q.dtype != torch.bfloat16 or D != 128:
                raise ValueError("pair_steps: bf16 with head_dim 128 (the MFMA step kernel)")
            if k_pool.shape[2] % 32:
                raise ValueError(f"pair_steps: the chunk length ({k_pool.shape[2]}) must be a multiple of 32")
            self.nbuf = max(1, self.cp - 1)
        chunk_shape = tuple(k_pool.shape[1:])
        dev = q.device
        self.kbuf = [torch.empty(chunk_shape, dtype=k_pool.dtype, device=dev) for _ in range(self.nbuf)]
        self.vbuf = [torch.empty(chunk_shape, dtype=v_pool.dtype, device=dev) for _ in range(self.nbuf)]
        self.copy_stream = copy_stream if copy_stream is not None else side_streams(2, dev)[0]
        self.copied = [torch.cuda.Event() for _ in range(self.cp)]
        self.consumed = [torch.cuda.Event() for _ in range(self.cp)]
        self.masks = [step_mask(layout, causal, rank, ring_source_rank(rank, s, self.cp)) for s in range(self.cp)]
        # the library splits key ranges only where query tiles alone would underfill the device
        nbytes = 0
        if split:
            nbytes = max(api.ring_attn_workspace_size(q.dtype, B, H, Sq, chunk_shape[1], D, m)
                         for m in set(x for x in self.masks if x is not None))
        if compute_streams is None:
            # const-max steps fold in order; split steps already fill the device
            compute_streams = 2 if (variant == "online" and not nbytes) else 1
        if variant == "constmax" and compute_streams > 1:
            raise ValueError("const-max steps add into one accumulator and run on one stream")
        self.aux_stream = side_streams(2, dev)[1] if compute_streams > 1 else None
        # one workspace per compute stream (concurrent steps may not share one)
        self.ws = [None, None]
        if nbytes:
            self.ws = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(compute_streams)]
            self.ws += [self.ws[0]] * (2 - len(self.ws))
        self.live_steps = [s for s in range(self.cp) if self.masks[s] is not None]
        assert self.live_steps, "a rank always sees its own chunk"
        self.fold = bool(fold)
        # one compute stream folding into an fp32 output needs no final merge
        self.fold_direct = self.fold and compute_streams == 1 and out_dtype == torch.float32
        if variant == "online":
            n = compute_streams if self.fold else len(self.live_steps)
            self.o_parts = torch.empty((max(n, 1), B, H, Sq, D), dtype=torch.float32, device=dev)
            self.lse_parts = torch.empty((max(n, 1), B, H, Sq), dtype=torch.float32, device=dev)
        else:
            self.kmax = torch.empty((B, H), dtype=torch.float32, device=dev)
            self.c = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
            self.acc = torch.empty(api.const_max_acc_size(B, H, Sq, D), dtype=torch.float32, device=dev)
        # sink-robust const-max: keys above sink_theta x the mean key norm leave the bound and
        # the fold, and are attended exactly in a second partial merged by LSE
        self.sink_theta = sink_theta if variant == "constmax" else None
        if self.sink_theta is not None:
            self.sinks = {"kmax_sq": torch.empty((B, H), dtype=torch.float32, device=dev),
                          "kmax_sq_robust": torch.empty((B, H), dtype=torch.float32, device=dev),
                          "knorm_sum": torch.empty((B, H), dtype=torch.float32, device=dev),
                          "sink_idx": torch.zeros((B, H, sink_cap), dtype=torch.int32, device=dev),
                          "sink_cnt": torch.empty((B, H), dtype=torch.int32, device=dev)}
            self.o_parts = torch.empty((2, B, H, Sq, D), dtype=torch.float32, device=dev)
            self.lse_parts = torch.empty((2, B, H, Sq), dtype=torch.float32, device=dev)
            self.sink_ws = torch.empty(max(16, api.sink_attention_workspace_size(B, H, D, sink_cap)),
                                       dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=dev)
        self.lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        self.step_events = None

    def _chunk(self, step):
        if step == 0:
            return self.k_pool[self.rank], self.v_pool[self.rank]
        j = (step - 1) % self.nbuf
        return self.kbuf[j], self.vbuf[j]

    def _issue_copy(self, step):
        src = ring_source_rank(self.rank, step, self.cp)
        kd, vd = self._chunk(step)
        with torch.cuda.stream(self.copy_stream):
            api.kv_chunk_copy(kd, vd, self.k_pool[src], self.v_pool[src])
            self.copied[step].record(self.copy_stream)

    def prologue(self):
        """const-max bound: per-head max key norm over the whole ring, then c per row (with
        sinks: the max over the non-sink keys, and the sink lists).
        With one sequence and a contiguous pool, the chunks are one [1, cp*S, H, D] run of
        keys and the max-fold over the ring is a single call."""
        kp = self.k_pool
        if self.sink_theta is not None:
            api.const_max_sink_prologue(kp, self.sink_theta, out=self.sinks)
            api.const_max_bound(self.q, self.sinks["kmax_sq_robust"], scale=self.scale, out=self.c)
            return
        if kp.shape[1] == 1 and kp.is_contiguous():
            cp, _, S, H, D = kp.shape
            api.key_sqnorm_max(kp.view(1, cp * S, H, D), self.kmax)
        else:
            for r in range(self.cp):
                api.key_sqnorm_max(kp[r], self.kmax, accumulate=r > 0)
        api.const_max_bound(self.q, self.kmax, scale=self.scale, out=self.c)

    def run(self, timing_events=None):
        """Runs the ring on the current stream; returns (out [B,H,Sq,D], lse [B,H,Sq]).
        ``timing_events``: optional list of cp (start, end) event pairs recorded around
        each step's kernel on the stream that runs it."""
        cs = torch.cuda.current_stream()
        cp = self.cp
        if self.pair_steps:
            return self._run_pairs(cs, timing_events)
        if self.fused_hops:
            return self._run_fused(cs, timing_events)
        if self.variant == "constmax":
            self.prologue()
        self.copy_stream.wait_stream(cs)
        if self.aux_stream is not None:
            self.aux_stream.wait_stream(cs)
        for t in range(1, min(self.depth, cp - 1) + 1):
            self._issue_copy(t)
        slot = 0
        started = [False, False]   # fold: running partial of each compute stream begun
        for s in range(cp):
            t = s + self.depth
            if s >= 1 and t < cp:
                # the buffer of step t was last read by step t - nbuf = s - 1
                self.copy_stream.wait_event(self.consumed[s - 1])
                self._issue_copy(t)
            second = self.aux_stream is not None and s % 2 == 1
            st = self.aux_stream if second else cs
            ws = self.ws[1 if second else 0]
            if s >= 1:
                st.wait_event(self.copied[s])
            k, v = self._chunk(s)
            with torch.cuda.stream(st):
                if timing_events is not None:
                    timing_events[s][0].record(st)
                if self.variant == "online":
                    if self.masks[s] is not None and self.fold:
                        a = 1 if second else 0
                        o_dst, l_dst = ((self.out, self.lse) if self.fold_direct
                                        else (self.o_parts[a], self.lse_parts[a]))
                        api.ring_attn_step(self.q, k, v, scale=self.scale, mask=self.masks[s], out=o_dst,
                                           lse=l_dst, workspace=ws, fold=started[a])
                        started[a] = True
                    elif self.masks[s] is not None:
                        api.ring_attn_step(self.q, k, v, scale=self.scale, mask=self.masks[s],
                                           out=self.o_parts[slot], lse=self.lse_parts[slot], workspace=ws)
                        slot += 1
                else:
                    phase = (api.CA_PHASE_INIT if s == 0 else 0) | (api.CA_PHASE_FINAL if s == cp - 1 else 0)
                    if self.sink_theta is None:
                        api.ring_attn_const_max_step(self.q, k, v, self.c, self.acc, phase, out=self.out,
                                                     lse=self.lse, scale=self.scale, workspace=ws)
                    else:
                        src = ring_source_rank(self.rank, s, cp)
                        api.ring_attn_const_max_step(self.q, k, v, self.c, self.acc, phase, out=self.o_parts[0],
                                                     lse=self.lse_parts[0], scale=self.scale, workspace=ws,
                                                     sinks=self.sinks, key_offset=src * k.shape[1])
                if timing_events is not None:
                    timing_events[s][1].record(st)
            self.consumed[s].record(st)
        if self.aux_stream is not None:
            cs.wait_stream(self.aux_stream)
        if self.variant == "online" and self.fold:
            if not self.fold_direct:
                n = 2 if started[1] else 1   # stream 0 always runs step 0, the rank's own chunk
                api.lse_merge(self.o_parts[:n], self.lse_parts[:n], out=self.out, lse_out=self.lse)
        elif self.variant == "online":
            api.lse_merge(self.o_parts[:slot], self.lse_parts[:slot], out=self.out, lse_out=self.lse)
        elif self.sink_theta is not None:
            api.sink_attention_partial(self.q, self.k_pool, self.v_pool, self.sinks, scale=self.scale,
                                       out=self.o_parts[1], lse=self.lse_parts[1], workspace=self.sink_ws)
            api.lse_merge(self.o_parts, self.lse_parts, out=self.out, lse_out=self.lse)
        # the copy stream must not run ahead into the next call's buffers
        cs.wait_stream(self.copy_stream)
        return self.out, self.lse


    def capture(self):
        """Captures one run() as a HIP graph (torch.cuda.CUDAGraph) and returns it; each
        replay() redoes the pass on the same inputs into self.out and self.lse. The pass
        launches only kernels and stream waits, no memset or allocation, so it captures as
        is. One eager pass first settles the library's lazy set-up outside the capture.
        Not offered for a pass with two compute streams and a copy stream (events joining all
        three): capturing one ended the process with a segmentation fault on this ROCm
        release, cause not found, so that form runs eagerly."""
        if self.aux_stream is not None and not self.fused_hops:
            raise NotImplementedError("capture: a pass with two compute streams and a copy stream is not captured; "
                                      "run it eagerly, or use one compute stream or fused_hops=True")
        cs = torch.cuda.current_stream()
        side = torch.cuda.Stream(device=self.q.device)
        side.wait_stream(cs)
        with torch.cuda.stream(side):
            self.run()
        cs.wait_stream(side)
        torch.cuda.synchronize(self.q.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        return g

    def _hop_buffers(self, t):
        kd, vd = self._chunk(t)
        src = ring_source_rank(self.rank, t, self.cp)
        return kd, vd, self.k_pool[src], self.v_pool[src]

    def _run_fused(self, cs, timing_events):
        """run() with every hop carried by a step call: step s also moves chunk s + 2 into its
        buffer (on the CUs the step leaves free, or just ahead of it), so no copy stream is
        used and the two compute streams never wait on each other. Chunk 1 is moved by a
        plain copy ahead of step 0 on the calling stream: beside step 0 it would share the
        device with a step that fills it (the Wan2.2 pass took 814 us that way, 797 us so)."""
        cp = self.cp
        if self.variant == "constmax":
            self.prologue()
        if cp > 1:
            api.kv_chunk_copy(*self._hop_buffers(1))
        if self.aux_stream is not None:
            self.aux_stream.wait_stream(cs)
        streams = [self.aux_stream if (self.aux_stream is not None and s % 2 == 1) else cs for s in range(cp)]
        slot = 0
        started = [False, False]   # fold: running partial of each compute stream begun
        for s in range(cp):
            st = streams[s]
            hop = self._hop_buffers(s + 2) if s + 2 < cp else None
            k, v = self._chunk(s)
            with torch.cuda.stream(st):
                if timing_events is not None:
                    timing_events[s][0].record(st)
                ws = self.ws[1 if st is not cs else 0]
                if self.variant == "constmax":
                    phase = (api.CA_PHASE_INIT if s == 0 else 0) | (api.CA_PHASE_FINAL if s == cp - 1 else 0)
                    api.ring_attn_const_max_step(self.q, k, v, self.c, self.acc, phase, out=self.out, lse=self.lse,
                                                 scale=self.scale, workspace=ws, hop=hop)
                elif self.masks[s] is not None and self.fold:
                    a = 1 if st is not cs else 0
                    o_dst, l_dst = ((self.out, self.lse) if self.fold_direct
                                    else (self.o_parts[a], self.lse_parts[a]))
                    api.ring_attn_step(self.q, k, v, scale=self.scale, mask=self.masks[s], out=o_dst, lse=l_dst,
                                       workspace=ws, fold=started[a], hop=hop)
                    started[a] = True
                elif self.masks[s] is not None:
                    api.ring_attn_step(self.q, k, v, scale=self.scale, mask=self.masks[s], out=self.o_parts[slot],
                                       lse=self.lse_parts[slot], workspace=ws, hop=hop)
                    slot += 1
                elif hop is not None:
                    api.kv_chunk_copy(*hop)
                if timing_events is not None:
                    timing_events[s][1].record(st)
        if self.aux_stream is not None:
            cs.wait_stream(self.aux_stream)
        if self.variant == "online" and self.fold:
            if not self.fold_direct:
                n = 2 if started[1] else 1   # stream 0 always runs step 0, the rank's own chunk
                api.lse_merge(self.o_parts[:n], self.lse_parts[:n], out=self.out, lse_out=self.lse)
        elif self.variant == "online":
            api.lse_merge(self.o_parts[:slot], self.lse_parts[:slot], out=self.out, lse_out=self.lse)
        return self.out, self.lse


    def _run_pairs(self, cs, timing_events):
        """run() with two steps per launch (ring_attn_step_pair). Launch i computes chunks
        2i and 2i + 1 on compute stream i % 2 and carries the hops of chunks 2i + 4 and
        2i + 5, which the next launch on the same stream reads. The chunks of each stream's
        first launch are copied ahead of it on that stream (chunk 1 before launch 0, chunks
        2 and 3 before launch 1, beside launch 0). Each received chunk has a buffer of its own,
        so no hop overwrites a chunk a launch on the other stream may still read."""
        cp = self.cp
        launches = [tuple(range(s, min(s + 2, cp))) for s in range(0, cp, 2)]
        aux = self.aux_stream
        streams = [aux if (aux is not None and i % 2 == 1) else cs for i in range(len(launches))]
        if aux is not None:
            aux.wait_stream(cs)
        for i in range(min(2, len(launches))):
            with torch.cuda.stream(streams[i]):
                for t in launches[i]:
                    if t >= 1:
                        api.kv_chunk_copy(*self._hop_buffers(t))
        started = [False, False]
        for i, chunks in enumerate(launches):
            st = streams[i]
            a = 0 if st is cs else 1
            hops = [self._hop_buffers(t) for t in (2 * i + 4, 2 * i + 5) if t < cp]
            o_dst, l_dst = self.o_parts[a], self.lse_parts[a]
            with torch.cuda.stream(st):
                if timing_events is not None:
                    for t in chunks:
                        timing_events[t][0].record(st)
                if len(chunks) == 2:
                    (k1, v1), (k2, v2) = self._chunk(chunks[0]), self._chunk(chunks[1])
                    api.ring_attn_step_pair(self.q, k1, v1, k2, v2, scale=self.scale, out=o_dst, lse=l_dst,
                                            workspace=self.ws[a], fold=started[a], hops=hops)
                else:
                    k, v = self._chunk(chunks[0])
                    api.ring_attn_step(self.q, k, v, scale=self.scale, out=o_dst, lse=l_dst, workspace=self.ws[a],
                                       fold=started[a], hop=hops[0] if hops else None)
                    for h in hops[1:]:
                        api.kv_chunk_copy(*h)
                if timing_events is not None:
                    for t in chunks:
                        timing_events[t][1].record(st)
            started[a] = True
        if aux is not None:
            cs.wait_stream(aux)
        n = 2 if started[1] else 1
        api.lse_merge(self.o_parts[:n], self.lse_parts[:n], out=self.out, lse_out=self.lse)
        return self.out, self.lse


def ring_attention(q_global, k_global, v_global, cp, rank, *, layout="contiguous", causal=False,
                   variant="online", scale=None, prefetch_depth=2, split=False, fold=False, compute_streams=None,
                   fused_hops=False, pair_steps=False):
    """Convenience: rank ``rank``'s output for global [B, S, H, D] inputs."""
    check_divisible(q_global.shape[1], cp)
    q = shard(q_global, cp, rank, layout)
    kp = chunk_pool(k_global, cp, layout)
    vp = chunk_pool(v_global, cp, layout)
    rp = RingPass(q, kp, vp, rank, layout=layout, causal=causal, variant=variant, scale=scale,
                  prefetch_depth=prefetch_depth, split=split, fold=fold, compute_streams=compute_streams,
                  fused_hops=fused_hops, pair_steps=pair_steps)
    return rp.run()
