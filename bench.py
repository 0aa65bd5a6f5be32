"""Decode-step benchmark of the CONF-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 384] [--warmup 128] [--workload NAME]

A step is one pass of the whole path over one batch: append + decode attention
(conf_attend), confidence + budgets (conf_confidence), and the EMA update, rank +
select and compaction + demotion in one launch (conf_ema_evict_compact), for
every layer and sequence.  HIP events around conf_attend time the attention
kernel alone.  Inputs (logits, q, k, v of every step) are
generated on the device before the timed region; the prefilled context is
ingested during set-up.  Default workload: the Qwen-32B-shaped GQA cache
(64 layers, 40 query / 8 KV heads, head_dim 128, bf16, batch 8, 32768-token
prefill with a planted needle, budgets 2048 / 4096, P 256, W 512).  The first
128 steps (the one-off bulk eviction of the prefill and the first confident /
unconfident phases) are warm-up; the timed steps are the steady state.

The confidence reads only the step's logits, and the selection is the first call
that needs its budgets, so on caches whose attention launch is long it runs on a
second stream (default priority) beside the attention; each step's second-stream
work is ordered after the previous step, and the selection waits for it.  On small
caches the two cross-stream waits per step cost more than they hide (measured:
the GPT-2-shaped caches ran 33-46% slower), so every call goes in order on one
stream.  --streams 1|2 overrides the choice.

On the same large caches the layers are split in two halves (two views of the one
cache, each with its own workspace), each half's attention and eviction in order on
a stream of its own and the two streams concurrent, so that one half's eviction
runs beside the other half's attention rather than after all of it (measured on the
Qwen-32B batch-8 cache: 0.494 against 0.540 ms per step; four or eight parts were
slower).  The attention time of a step is then the union of its two launches, from
the first start to the last end, and the roofline's bytes are those of all layers.
Only caches whose attention launch has at least 2048 workgroups and whose K/V at the
tight budget, counted at one byte per channel, reach 512 MiB per step are split (the
Qwen-32B batch-1 cache, 512 workgroups, fell to 0.55x; the 256-token sliding-window
baselines of the Qwen-14B and gpt-oss-20b shapes, 384 MiB, to 0.55-0.69x).  --split
1|2 overrides the choice.

A half's attention of step s+1 waits for that half's eviction of step s and for
nothing of the other half, so successive steps overlap across the halves: every
cache is read only after its own eviction, but a step's first layers start before
the previous step's last layers end, which a model's forward pass, one layer after
another, would not allow (there, each layer's eviction would run beside the
model's later layers instead).  --strict-steps makes every launch of a step wait
for all of the previous step (measured: 10-14% fewer steps/s on the split caches,
the attention's rate about unchanged); the line's config says which ran
(steps_overlap).

--policy full | window runs the same step under the full-KV or the sliding-window
baseline (the pages' comparison policies) on the same kernels and shape: full KV
keeps every prefill and decoded token in 16 bits, the window the newest W.
--policy arkv runs ARKV's three-state cache: a step is the attention and the ARKV
launches (score EMA, eviction to N = N_high, quantisation to e4m3 of the lowest-
ranked Original tokens beyond the layer's N_O), with no confidence.
--policy trim runs retention eviction: a step is the attention and one launch that
stores the new token's ln(beta), ranks by (t - pos) * ln(beta) and compacts, with a
16-bit cache of M = N_high tokens (the prefill cut to M) and no confidence.

Besides the steady-state figures, the JSON line reports step0_ms, the one-off first
step after the prefill (the cut of the prefilled cache to its budget), timed on its
own during warm-up (after one step of a one-layer copy of the workload and a first
use of every stream, so that it holds the step's work and not the process's first
kernel launches or queue set-up), and copy_ceiling_GBs, the best rate of a plain 2 GiB device copy
on the same box (bytes read + written), as a measured ceiling next to the nominal
8 TB/s.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import contextlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from adaptive_kv_cache_amd import synth  # noqa: E402
from adaptive_kv_cache_amd.binding import Engine  # noqa: E402
from adaptive_kv_cache_amd.workloads import WORKLOADS  # noqa: E402

METRIC = "decode steps/s (attn+confidence+evict+compact), HBM GB/s vs peak, batch 8"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- byte model
def _heads(wl):
    """KV heads per cache: one when each head keeps its own tokens."""
    return 1 if wl.headwise else wl.n_kv_heads


def _qheads(wl):
    return wl.group if wl.headwise else wl.n_q_heads


def attn_bytes(wl, n8, nw):
    """Algorithmic bytes of one attention launch (conf_attend: every layer and
    sequence; the EMA update is counted with the step).

    n8, nw: int64 tensors [L][B] of INT8 and window tokens before the append
    ([L][B*Hkv] head-wise, each cache then holding one KV head).
    Per (layer, sequence): cached K and V (1 byte per INT8 element, e per 16-bit
    element), this step's k and v read and appended, both absmax rows, and q in
    and o out (fp32).
    """
    e = 2
    H, d, Hq = _heads(wl), wl.head_dim, _qheads(wl)
    kv = 2 * H * d * (n8 + e * nw)
    per_lb = kv + 2 * H * d * e * 2 + 2 * H * d * 4 + Hq * d * (e + 4)
    return int(per_lb.sum())


def step_bytes(wl, n8, nw, plan):
    """Algorithmic bytes of one whole step: attention, logits, the EMA update, the
    selection's position reads, hole-fill moves and the demotion (requantisation
    not counted; the selection takes the EMA it has just written, and the keep
    flags stay on chip in the fused EMA + selection + compaction launch).  The
    baselines read what their policy needs: full KV ranks nothing, the window
    reads positions, retention eviction reads ln(beta) and positions and has no
    confidence."""
    H, d, e = _heads(wl), wl.head_dim, 2
    n = n8 + nw + 1
    b = attn_bytes(wl, n8, nw)
    if wl.policy not in ("trim", "arkv"):
        b += wl.batch * wl.vocab * 4                            # logits (confidence)
    if wl.policy in ("confkv", "arkv"):
        b += int((8 * n + 4).sum())                             # EMA read and written, new pos
    else:
        b += 8 * n.numel()                                      # the new token's EMA slot and pos
    if wl.policy == "trim":
        b += int((4 * n).sum())                                 # ln(beta) read by the ranking
    if wl.policy != "full":
        b += int((4 * n).sum())                                 # positions read by the selection
    moves8, moves16, dest = plan[..., 1], plan[..., 3], plan[..., 5]
    b += int((moves8 * (2 * 2 * H * d + 16)).sum())
    b += int((moves16 * (2 * 2 * H * d * e + 16)).sum())
    b += int(((dest >= 0).long() * (2 * H * d * (e + 1) + 8)).sum())
    return b


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, seed, n_tokens, first_step, budget_s=20.0):
    """The oracle as it stands, on a bounded sample of the timed regime: every
    layer of one sequence, stepped from a cache of the size the timed GPU steps
    attended (n_tokens - 1 cached tokens plus the appended one) with the logits of
    the timed steps from `first_step` on, for as many steps as fit in about
    `budget_s`."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    cores = len(os.sched_getaffinity(0))
    prm = O.OracleParams(n_layers=wl.n_layers, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                         head_dim=wl.head_dim, dtype16=wl.dtype16, window=wl.window,
                         protect=wl.protect, n_high=wl.n_high, n_low=wl.n_low,
                         pyramid=wl.pyramid, tau=wl.tau)
    n0 = max(1, int(round(n_tokens)) - 1)
    rng = np.random.default_rng(seed)
    states = []
    for l in range(wl.n_layers):
        k = O.encode16(rng.standard_normal((wl.n_kv_heads, n0, wl.head_dim)), wl.dtype16)
        v = O.encode16(rng.standard_normal((wl.n_kv_heads, n0, wl.head_dim)), wl.dtype16)
        states.append([O.ingest(k, v, wl.window, wl.dtype16)])
    steps = 0
    t0 = time.perf_counter()
    while True:
        z = synth.logits(wl.scaled(batch=1), first_step + steps, seed).numpy().astype(np.float64)
        q = O.encode16(rng.standard_normal((wl.n_layers, 1, wl.n_q_heads, wl.head_dim)),
                       wl.dtype16)
        kk = O.encode16(rng.standard_normal((wl.n_layers, 1, wl.n_kv_heads, wl.head_dim)),
                        wl.dtype16)
        vv = O.encode16(rng.standard_normal((wl.n_layers, 1, wl.n_kv_heads, wl.head_dim)),
                        wl.dtype16)
        O.decode_step(states, z, q, kk, vv, prm)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 64:
            break
    per_seq_step = el / steps
    return {
        "value": 1.0 / (per_seq_step * wl.batch), "unit": "steps/s", "cores": cores,
        "blas_threads": blas, "kind": "oracle",
        "sample": (f"{steps} steps x {wl.n_layers} layers x 1 sequence from a {n0 + 1}-token "
                   f"cache (the timed steps' mean), logits of steps {first_step}.."
                   f"{first_step + steps - 1}; {per_seq_step:.3f} s per sequence-step, "
                   f"extrapolated to batch {wl.batch}"),
    }


# ---------------------------------------------------------------- GPU run
def prime_kernels(wl, dev, seed):
    """One decode step of a one-layer, one-sequence copy of the workload (same head
    shape, precision and policy, a shorter prefill), so that every kernel the step
    launches has been launched once in this process before step 0 is timed: a
    kernel's first launch loads its code and sets its attributes, a one-off cost of
    the process rather than of the step."""
    small = wl.scaled(n_layers=1, batch=1,
                      prefill=min(wl.prefill, 2 * (wl.n_low + wl.window)) if wl.prefill else 0)
    e = Engine(small, dev)
    if small.prefill:
        k, v = synth.prefill_kv(small, 0, seed, device=dev)
        e.ingest(0, k, v)
        if small.policy == "arkv":
            conc = e.arkv_prefill_stats(0, synth.q_new(small, 0, seed, device=dev)[0], k)
        if small.policy == "trim":
            e.set_retention(0, synth.log_beta_prefill(small, 0, seed, device=dev))
    q = synth.q_new(small, 0, seed, device=dev)
    k, v = synth.kv_new(small, 0, seed, device=dev)
    e.attend(-1, q, k, v)
    if small.policy == "trim":
        e.trim_evict_compact(-1, torch.full((1, 1), small.n_high, dtype=torch.int32, device=dev),
                             synth.log_beta_new(small, 0, seed, device=dev))
    elif small.policy == "arkv":
        budget = torch.full((1, 1), small.n_high, dtype=torch.int32, device=dev)
        n_orig = e.arkv_orig_budgets(conc) if small.prefill else budget.clone()
        e.arkv_ema_evict_compact(-1, budget, n_orig)
    else:
        _, budget = e.confidence(synth.logits(small, 0, seed, device=dev))
        e.ema_evict_compact(-1, budget)
    torch.cuda.synchronize()
    del e
    torch.cuda.empty_cache()


def run(args):
    wl = WORKLOADS[args.workload].baseline(args.policy, args.warmup + args.steps)
    if args.headwise:
        wl = wl.headwise_variant()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    total = args.warmup + args.steps
    if total > wl.steps:
        log(f"note: {total} steps exceed the workload's {wl.steps}; inputs are generated anyway")
    log(f"set-up {wl.name}: cap8={wl.cap8} prefill={wl.prefill}")
    prime_kernels(wl, dev, args.seed)
    eng = Engine(wl, dev)
    trim = wl.policy == "trim"
    arkv = wl.policy == "arkv"
    no_conf = trim or arkv  # these policies take no confidence-chosen budget
    t0 = time.perf_counter()
    ingest_ms = 0.0
    if wl.policy == "arkv":
        # ARKV's prefill phase: the first decode step's queries over each layer's prefill
        # keys give the layers' concentrations, from which their Original budgets follow
        q0 = synth.q_new(wl, 0, args.seed, device=dev)
        conc = torch.zeros(wl.n_layers, wl.batch, dtype=torch.float32, device=dev)
    if wl.prefill:
        for l in range(wl.n_layers):
            k, v = synth.prefill_kv(wl, l, args.seed, device=dev)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            eng.ingest(l, k, v)
            b.record()
            if wl.policy == "arkv":
                eng.arkv_prefill_stats(l, q0[l], k, conc)
            if trim:
                eng.set_retention(l, synth.log_beta_prefill(wl, l, args.seed, device=dev))
            b.synchronize()
            ingest_ms += a.elapsed_time(b)
            del k, v
    torch.cuda.synchronize()
    log(f"ingest done in {time.perf_counter() - t0:.1f} s (conf_cache_ingest {ingest_ms:.1f} ms)")
    L, B = wl.n_layers, wl.batch
    logits = torch.empty(total, B, wl.vocab, dtype=torch.float32, device=dev)
    qs = torch.empty(total, L, B, wl.n_q_heads, wl.head_dim, dtype=eng.dtype16, device=dev)
    ks = torch.empty(total, L, B, wl.n_kv_heads, wl.head_dim, dtype=eng.dtype16, device=dev)
    vs = torch.empty_like(ks)
    for s in range(total):
        logits[s] = synth.logits(wl, s, args.seed, device=dev)
        qs[s] = synth.q_new(wl, s, args.seed, device=dev)
        ks[s], vs[s] = synth.kv_new(wl, s, args.seed, device=dev)
    if trim:
        # retention eviction: ln(beta) of each new token, and the memory budget M
        lbetas = torch.stack([synth.log_beta_new(wl, s, args.seed, device=dev)
                              for s in range(total)])
    out = torch.empty(L, B, wl.n_q_heads, wl.head_dim, dtype=torch.float32, device=dev)
    conf = torch.empty(total, B, dtype=torch.float32, device=dev)
    budget = torch.empty(total, B, L, dtype=torch.int32, device=dev)
    if no_conf:
        budget.fill_(wl.n_high)
    if arkv:
        # ARKV: N = N_high kept tokens, N_O of them Original per the layer's OQ ratio
        # from its prefill attention statistics
        n_orig = eng.arkv_orig_budgets(conc)
    S = wl.n_sub
    n8_first = torch.empty(L, S, dtype=torch.int32, device=dev)
    n16_first = torch.empty_like(n8_first)
    hplan = torch.empty(args.steps, L, S, 16, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream(dev)
    # K/V bytes of one step's attention at the tight budget, counted at one byte per
    # channel: the split and the second stream pay from 512 MiB (measured: the CONF-KV
    # Qwen-14B and gpt-oss-20b caches, 960 MiB by this count, gain from the halves;
    # their 256-token sliding-window baselines, 384 MiB, ran 0.55-0.69x with them)
    big = L * B * wl.n_kv_heads * wl.head_dim * (wl.n_high + wl.window) * 2 >= 1 << 29
    streams = args.streams
    if streams == "auto":
        # nothing to overlap otherwise; in a graph the confidence branch costs no launch
        streams = "2" if (big or args.graph) and not no_conf else "1"
    side = main if streams == "1" else torch.cuda.Stream(device=dev)
    split = args.split
    if split == "auto":
        # halves of at least 1024 workgroups each (four per compute unit); smaller
        # launches lose more to the extra launches and waits than the overlap gains
        # (measured: the Qwen-32B batch-1 cache, 512 units, fell from 8476 to 4684 steps/s)
        units = L * B * wl.n_kv_heads
        split = "2" if big and units >= 2048 else "1"
    split = int(split)
    if args.graph and split != 1:
        raise SystemExit("--graph captures one layer range: use --split 1 (or auto on a small cache)")
    if split > 1 and side is main:
        side = torch.cuda.Stream(device=dev)  # the halves must not wait on each other
    # Layer halves: two views of the one cache, each with its own workspace, each
    # half's attention and eviction in order on a stream of its own, the two
    # streams concurrent.  A half's eviction then runs beside the other half's
    # attention instead of after all of it.
    ranges = [(i * L // split, (i + 1) * L // split) for i in range(split)]
    views = [eng] if split == 1 else [eng.layer_view(a, b - a) for a, b in ranges]
    vstreams = [main] + [torch.cuda.Stream(device=dev) for _ in range(split - 1)]
    ws_plans = []
    for v, (a, b) in zip(views, ranges):
        off = _plan_offset(v)
        ws_plans.append(v.ws[off:off + (b - a) * S * 16 * 4].view(torch.int32).view(b - a, S, 16))
    # per-view budget columns (copied after the confidence), ln(beta) rows, N_O columns
    bsl = [budget[:, :, a:b].clone() for a, b in ranges] if split > 1 else [budget]
    norig_v = [n_orig[:, a:b].contiguous() for a, b in ranges] if arkv else None
    # every step's per-view arguments, sliced once here: on the launch-bound caches the
    # Python between a launch's start event and the launch is part of what is timed
    if split == 1:
        vargs = [[(qs[s], ks[s], vs[s], out, budget[s], lbetas[s] if trim else None)]
                 for s in range(total)]
    else:
        vargs = [[(qs[s][a:b], ks[s][a:b], vs[s][a:b], out[a:b], bsl[k][s],
                   lbetas[s][a:b] if trim else None) for k, (a, b) in enumerate(ranges)]
                 for s in range(total)]
    # a stream's first use sets up its hardware queue: done here, not inside step 0
    for st in {id(x): x for x in vstreams + [side]}.values():
        with torch.cuda.stream(st):
            torch.zeros(1, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident; warm-up (streams {streams}, layer split {split})")

    def one_step(s, ev=None, i=None):
        for st in vstreams:
            if side is not st:
                side.wait_stream(st)
        if args.strict_steps:  # every launch of step s after all of step s-1
            for st in vstreams:
                for o in vstreams + [side]:
                    if o is not st:
                        st.wait_stream(o)
        with torch.cuda.stream(side):
            # bookkeeping for the byte model: the previous timed step's compaction
            # plans, copied while the attention runs (the compactions that overwrite
            # them wait for this stream)
            if i:
                for (a, b), wp in zip(ranges, ws_plans):
                    hplan[i - 1, a:b].copy_(wp)
            if not no_conf:
                eng.confidence(logits[s], c=conf[s], budget=budget[s])
                if split > 1:
                    for (a, b), t in zip(ranges, bsl):
                        t[s].copy_(budget[s][:, a:b])
        for k, (v, st, (q_, k_, v_, o_, b_, lb_)) in enumerate(zip(views, vstreams, vargs[s])):
            with (torch.cuda.stream(st) if st is not main else contextlib.nullcontext()):
                if ev is not None:
                    ev[2 * k].record(st)
                v.attend(-1, q_, k_, v_, out=o_)
                if ev is not None:
                    ev[2 * k + 1].record(st)
                if side is not st:
                    st.wait_stream(side)
                if trim:
                    v.trim_evict_compact(-1, b_, lb_)
                elif arkv:
                    v.arkv_ema_evict_compact(-1, b_, norig_v[k])
                else:
                    v.ema_evict_compact(-1, b_)

    step0 = None
    for s in range(args.warmup):
        if s == 0:  # the one-off step after the prefill, timed on its own
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        one_step(s)
        if s == 0:
            for st in vstreams[1:]:
                main.wait_stream(st)
            main.wait_stream(side)
            e1.record()
            torch.cuda.synchronize()
            step0 = e0.elapsed_time(e1)
        if s % 32 == 0:
            torch.cuda.synchronize()
            log(f"  warm-up step {s}")
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * split)]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timed: {args.steps} steps")
    # the sizes before the first timed step; later ones follow from each step's plan
    n8_first.copy_(eng.t_n8)
    n16_first.copy_(eng.t_n16)
    torch.cuda.synchronize()
    if args.graph:
        # every timed step captured in one HIP graph (kernel nodes, and the plan
        # copies of the byte model as copy nodes), replayed once in the timed region;
        # with a second stream each step's confidence is a branch beside its
        # attention, joined before its eviction
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                s = args.warmup + i
                q_, k_, v_, o_, b_, lb_ = vargs[s][0]
                if i:
                    hplan[i - 1].copy_(ws_plans[0])
                fork = not no_conf and side is not main
                if fork:
                    side.wait_stream(cap)
                    with torch.cuda.stream(side):
                        eng.confidence(logits[s], c=conf[s], budget=budget[s])
                eng.attend(-1, q_, k_, v_, out=o_)
                if trim:
                    eng.trim_evict_compact(-1, b_, lb_)
                elif arkv:
                    eng.arkv_ema_evict_compact(-1, b_, norig_v[0])
                else:
                    if fork:
                        cap.wait_stream(side)
                    else:
                        eng.confidence(logits[s], c=conf[s], budget=budget[s])
                    eng.ema_evict_compact(-1, b_)
        torch.cuda.synchronize()
        start.record()
        graph.replay()
        end.record()
    else:
        start.record()
        for st in vstreams[1:]:
            st.wait_event(start)
        for i in range(args.steps):
            one_step(args.warmup + i, evs[i], i)
        for st in vstreams[1:]:
            main.wait_stream(st)
        end.record()
    for (a, b), wp in zip(ranges, ws_plans):
        hplan[args.steps - 1, a:b].copy_(wp)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    # attention-busy time: the union of every attention launch's [start, end] over the
    # timed region (one launch per step: the sum of their durations; with layer parts
    # on concurrent streams the launches of a step, and of successive steps, overlap)
    if args.graph:
        # no per-launch events inside a graph: the whole step time bounds the
        # attention's (its rate below is then a lower bound)
        attn_ms = [ms / args.steps]
    else:
        spans = sorted((start.elapsed_time(e[2 * k]), start.elapsed_time(e[2 * k + 1]))
                       for e in evs for k in range(split))
        busy, cur0, cur1 = 0.0, None, None
        for a0, a1 in spans:
            if cur1 is None or a0 > cur1:
                busy += 0.0 if cur1 is None else cur1 - cur0
                cur0, cur1 = a0, a1
            else:
                cur1 = max(cur1, a1)
        busy += cur1 - cur0
        attn_ms = [busy / args.steps]
    st = eng.status()
    if st:
        raise RuntimeError(f"cache status word {st}: a capacity was exceeded")
    hp = hplan.cpu().long()
    # sizes after each step: n8 = plan n8' (+1 if a token was demoted), n16 = plan n16'
    n8_after = hp[..., 0] + (hp[..., 5] >= 0).long()
    n16_after = hp[..., 2]
    # the plan copied from the workspace must describe the cache the last step left
    if not (torch.equal(n8_after[-1], eng.t_n8.cpu().long())
            and torch.equal(n16_after[-1], eng.t_n16.cpu().long())):
        raise RuntimeError("workspace plan offset does not match the library's layout")
    h8 = torch.cat([n8_first.cpu().long()[None], n8_after[:-1]])
    h16 = torch.cat([n16_first.cpu().long()[None], n16_after[:-1]])
    a_bytes = [attn_bytes(wl, h8[i], h16[i]) for i in range(args.steps)]
    s_bytes = [step_bytes(wl, h8[i], h16[i], hp[i]) for i in range(args.steps)]
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    attn_gbs = (sum(a_bytes) / len(a_bytes)) / (attn_avg_ms * 1e-3) / 1e9
    sps = args.steps / (ms * 1e-3)
    step_gbs = (sum(s_bytes) / len(s_bytes)) * sps / 1e9
    n_mean = float((h8 + h16 + 1).float().mean())
    res = {
        "metric": METRIC, "value": round(sps, 3), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ({"confkv": f"int8+{wl.dtype16}", "arkv": f"fp8(e4m3)+{wl.dtype16}"}
                  .get(wl.policy, wl.dtype16) + " operands, f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": wl.name, "policy": wl.policy, "headwise": wl.headwise,
                   "layers": L, "batch": B,
                   "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "dtype16": wl.dtype16,
                   "prefill": wl.prefill, "n_high": wl.n_high, "n_low": wl.n_low,
                   "protect": wl.protect, "window": wl.window, "pyramid": wl.pyramid,
                   "vocab": wl.vocab, "mean_tokens_attended": round(n_mean, 1),
                   "streams": 1 + (split - 1) + (side is not main), "layer_split": split,
                   "steps_overlap": split > 1 and not args.strict_steps,
                   "graph": bool(args.graph)},
        "roofline": {"bound": "hbm",
                     "kernel": "attn_kernel (conf_attend; " +
                               ("graph replay of every timed step: duration = the whole step, so "
                                "the rate is a lower bound)" if args.graph else
                                "one launch per step)" if split == 1 else
                                f"{split} concurrent launches per step over layer ranges; "
                                "duration = attention-busy time per step, the union of all "
                                "launch intervals)"),
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(wl.name, args.steps, args.warmup,
                                                round(n_mean, 1)),
                     "avg_launch_us": round(attn_avg_ms * 1e3, 2),
                     "alg_bytes_per_launch": int(sum(a_bytes) / len(a_bytes))},
        "step_roofline": {"achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                          "alg_bytes_per_step": int(sum(s_bytes) / len(s_bytes))},
        "step0_ms": None if step0 is None else round(step0, 3),
        "budgets": None if no_conf else budget_stats(budget[args.warmup:total, :, 0].cpu(), wl),
        "arkv_n_orig": None if not arkv else {
            "min": int(n_orig.min()), "max": int(n_orig.max()),
            "mean": round(float(n_orig.float().mean()), 1), "of_N": wl.n_high},
        "copy_ceiling_GBs": round(copy_ceiling(dev), 1),
        "ingest": ingest_stats(wl, ingest_ms) if wl.prefill else None,
    }
    return res, wl


def ingest_stats(wl, ms):
    """conf_cache_ingest over every layer: time and algorithmic bytes (the 16-bit
    prefill read once, the 8-bit codes and the window written).  The kernels read
    the INT8 part of the prefill twice, once for the absmax and once for the codes."""
    units = wl.n_layers * wl.batch * wl.n_kv_heads
    old = max(0, wl.prefill - wl.window)
    n8 = 0 if wl.policy == "window" else old
    nw = wl.prefill - old
    byts = units * wl.head_dim * (2 * 2 * (n8 + nw) + 2 * n8 + 2 * 2 * nw)
    return {"ms": round(ms, 2), "bytes": byts, "GBs": round(byts / (ms * 1e-3) / 1e9, 1)}


def budget_stats(b0, wl):
    """Budgets the confidence chose in the timed steps (layer 0's column [steps][B]):
    the fraction of (step, sequence) pairs on the tight budget N_high, and the
    fraction of sequences whose budget changed from one timed step to the next."""
    b0 = b0.long()
    flips = float((b0[1:] != b0[:-1]).float().mean()) if b0.shape[0] > 1 else 0.0
    return {"confident_fraction": round(float((b0 == wl.n_high).float().mean()), 4),
            "flip_rate": round(flips, 4)}


def _plan_offset(eng):
    """Byte offset of the compaction plan inside the workspace (same arithmetic
    as the library's workspace map: 256-byte aligned regions in a fixed order)."""
    wl = eng.wl
    LB = wl.n_layers * wl.n_sub
    a = lambda x: (x + 255) & ~255  # noqa: E731
    nch = -(-wl.vocab // (256 * 16))
    off = a(wl.n_sub * nch * 8 * 4)
    off = a(off + LB * _heads(wl) * (eng.cap8 + eng.cap16) * 4)
    off = a(off + LB * (eng.cap8 + eng.cap16))
    return off


def rocpd_summary(db_path, timed_steps, split=1):
    """Per-kernel durations from a rocprofv3 database of a bench run: every
    dispatch, and the last `timed_steps * split` dispatches of each kernel (the
    timed steady-state steps when the kernel runs once per step and layer part);
    with split > 1 also the attention's union per step."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration from kernels order by start").fetchall()
    per = {}
    for name, dur in rows:
        short = name.split("(")[0].replace("void ", "").replace("confkv::", "")
        per.setdefault(short[:70], []).append(dur)
    lines = [f"rocpd database: {os.path.basename(db_path)}",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>10s} "
             f"{'last' + str(timed_steps) + '_avg_us':>14s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        tail = v[-timed_steps * split:]
        lines.append(f"{k:70s} {len(v):6d} {sum(v) / len(v) / 1e3:10.2f} {min(v) / 1e3:9.2f} "
                     f"{max(v) / 1e3:10.2f} {sum(tail) / len(tail) / 1e3:14.2f}")
    # attention-busy time per step: the union of the last timed_steps * split
    # attention dispatch intervals, divided by timed_steps
    att = db.execute("select start, end from kernels where name like '%attn_kernel%' "
                     "order by start").fetchall()[-timed_steps * split:]
    if att:
        busy, c0, c1 = 0, None, None
        for a0, a1 in att:
            if c1 is None or a0 > c1:
                busy += 0 if c1 is None else c1 - c0
                c0, c1 = a0, a1
            else:
                c1 = max(c1, a1)
        busy += c1 - c0
        lines.append(f"attn_kernel busy time per step (union of the last {len(att)} dispatch "
                     f"intervals / {timed_steps}): {busy / timed_steps / 1e3:.2f} us")
    return "\n".join(lines)


# ---------------------------------------------------------------- counters
PROFILES = os.path.join(ROOT, "profiles")  # counter summaries: attn_traffic_*.md
ATTN_SOURCES = ("adaptive_kv_cache_amd/csrc/k_attn.hip", "adaptive_kv_cache_amd/csrc/common.hpp")


def attn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, steps, warmup, tokens):
    """HBM bytes per attention launch (one step's attention) from the committed
    counter summary, for exactly this regime: the same workload, timed steps,
    warm-up steps and mean tokens attended (the 4097-token phase after the prefill
    and the 2065-token steady state stream different bytes), on the same attention
    sources.  None when no such line exists."""
    try:
        names = sorted(f for f in os.listdir(PROFILES)
                       if f.startswith("attn_traffic_") and f.endswith(".md"))
    except OSError:
        return None
    want = {"workload": workload, "steps": str(steps), "warmup": str(warmup),
            "tokens": f"{tokens:.1f}", "source": attn_source_hash()}
    for name in names:
        with open(os.path.join(PROFILES, name)) as fh:
            text = fh.read()
        for line in text.splitlines():
            if not line.startswith("traffic:"):
                continue
            vals = dict(kv.partition("=")[::2] for kv in line[len("traffic:"):].split())
            if all(vals.get(k) == v for k, v in want.items()):
                return int(vals["bytes_per_launch"])
    return None


def copy_ceiling(dev, mib=2048, reps=8):
    """Measured HBM ceiling on this machine: a plain device copy (torch.neg, one read
    and one write of `mib` MiB per launch), best of `reps` launches, in GB/s of
    bytes read + written."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, device=dev).uniform_()
    dst = torch.empty_like(src)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.neg(src, out=dst)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (best * 1e-3) / 1e9


def copy_calibration(mib, reps):
    """A plain copy kernel of known size (reads and writes `mib` MiB each time), run
    under a counter pass to scale FETCH_SIZE / WRITE_SIZE to bytes."""
    dev = torch.device("cuda", 0)
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "reps": reps}))


def pmc_summary(csv_path, last):
    """Mean counter value per dispatch of each kernel (its last `last` dispatches)
    from a rocprofv3 --pmc counter_collection.csv."""
    import csv
    per = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            name = row["Kernel_Name"].split("(")[0].replace("void ", "").replace("confkv::", "")
            per.setdefault((name[:70], row["Counter_Name"]), []).append(float(row["Counter_Value"]))
    lines = [f"{'kernel':70s} {'counter':12s} {'dispatches':>10s} {'mean_last':>14s}"]
    for (k, ctr), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        tail = v[-last:]
        lines.append(f"{k:70s} {ctr:12s} {len(v):10d} {sum(tail) / len(tail):14.1f}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=384)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="qwen32b_gqa_b8_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--policy", choices=("confkv", "full", "window", "trim", "arkv"),
                    default="confkv",
                    help="cache policy: CONF-KV, or the full-KV / sliding-window / retention-"
                         "eviction / ARKV baseline on the same kernels")
    ap.add_argument("--headwise", action="store_true",
                    help="head-wise keep sets: each KV head keeps its own tokens, the layer's "
                         "Hkv * N pairs shared by the heads")
    ap.add_argument("--split", choices=("auto", "1", "2"), default="auto",
                    help="2: the layers in two halves on two concurrent streams, each half's "
                         "eviction beside the other half's attention; auto: 2 when the "
                         "attention streams at least 256 MB per step")
    ap.add_argument("--strict-steps", action="store_true",
                    help="with the layer halves: every launch of a step waits for all of the "
                         "previous step (by default a half's next attention waits only for its "
                         "own eviction, so successive steps overlap across the halves)")
    ap.add_argument("--streams", choices=("auto", "1", "2"), default="auto",
                    help="2: confidence on a second stream beside the attention; auto: 2 when "
                         "the attention streams at least 256 MB per launch")
    ap.add_argument("--graph", action="store_true",
                    help="capture every timed step in one HIP graph and replay it (no layer "
                         "split; the confidence a branch beside the attention unless --streams 1: "
                         "for the launch-bound small caches)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--rocpd-summary", metavar="DB",
                    help="print per-kernel durations of a rocprofv3 database and exit")
    ap.add_argument("--pmc-summary", metavar="CSV",
                    help="print per-kernel mean counter values of a rocprofv3 --pmc csv and exit")
    ap.add_argument("--copy-calibration", metavar="MIB", type=int,
                    help="run a plain copy kernel of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.rocpd_summary:
        print(rocpd_summary(args.rocpd_summary, args.steps, 1 if args.split == "auto"
                            else int(args.split)))
        return
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary, args.steps))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 8)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described in the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    res, wl = run(args)
    if not args.no_cpu_baseline and args.policy == "confkv" and not args.headwise:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(wl, args.seed,
                                           res["config"]["mean_tokens_attended"], args.warmup,
                                           args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
