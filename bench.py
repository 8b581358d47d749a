"""Benchmark: one Hash-sparse SCFA training step per iteration on one MI355X.

Workload (synthetic, seeded): B=2, H=12, T=16384, d=64, 32 LSH buckets,
block 64, bf16 -- the GPT-2-small attention shape at 16k tokens.  One step is
the whole hot path over one batch, with every input already in HBM:

  LSH bucket ids + (bucket, position) sort of Q and of K (one call over the
  two stacked in one [2B, H, T, d] allocation), block metadata (row and
  column live-tile lists), forward, backward dQ (+ rowsum(dO*O)), backward
  dK/dV; the attention kernels read Q, dO, K and V through the sort
  permutations (--copy-sorted: the sorts copy Q with dO and K with V into
  sorted order instead, in two calls).

Reported value: effective TFLOP/s on executed tiles (forward 4*bq*bk*d and
backward 10*bq*bk*d flops per executed tile of real extent bq x bk) over the
whole step.  Also reported: the same library's dense causal forward+backward
at the original shape and the speedup over it, per-kernel HIP-event times, the
roofline of the dominant kernel, and the CPU oracle on a bounded sample.  The
dense-causal comparator is timed at every block size the kernels take (64 and
128) and the faster is kept, in every line and sweep that quotes a speedup.

Timing starts after W untimed steps (default 60): the first few tens of
milliseconds of work run at lower clocks, about 12 % slower per step here.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-dense] [--copy-calibration MIB]
       python bench.py --sweep-nb 2,4,8,16,32,64,128 [--steps K] [--warmup W]
       python bench.py --measure-rows [--steps K] [--warmup W]
       python bench.py --sweep-drop 0,0.1,...,0.9 | --sweep-T 1024,...,1048576 [--steps K]

--sweep-drop: QK-sparse training step (B=4, H=12, T=8192, d=64) at each drop
rate: compaction (gather), forward + backward on the kept tokens,
un-compaction (scatter), against two naive ways of dropping tokens (the
compacted tensors with every tile computed and then masked; full-length
causal attention with the dropped tokens masked by position) and against
dense causal attention with nothing dropped.
--sweep-T: Hash-sparse (B=1, H=8, d=64, 32 buckets) at each length: LSH +
sort of Q and K, forward + backward; up to 32k tokens also the dense-causal
step and the naive hash attention (every tile computed, then masked:
NO_PRUNE + FORCE_MASK on the same sorted inputs); beyond, forward only.
Both print one JSON line per point (synthetic inputs drawn on the GPU).

--measure-rows times the row gather / scatter calls around the path at the
same shape (un-sorting O, dQ, dK, dV of the step; compacting Q, K, V to a
70% kept set) and prints one JSON line with their HBM throughput.

--sweep-nb runs the same step at the same shape for each bucket count and
prints one JSON line per count (executed tiles, step time, effective TFLOP/s,
speedup over the dense-causal path with and without the LSH + sort), then the
dense-causal reference line; it is a measurement mode, not the benchmark line.

HBM traffic of the dominant kernel ("roofline.traffic") comes from rocprofv3
FETCH_SIZE / WRITE_SIZE counter runs summarised under profiles/, scaled by
what the same counters read for a plain device copy of known size
(--copy-calibration makes this process run one, before the warmup).  The
summary records a digest of the kernel's sources and build flags; once they
change, traffic is reported as null until the counters are taken again.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E (published)
PEAK_FP64_TFLOPS = 78.6  # MI355X fp64 vector (published)
WORKLOAD_ID = 4
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_bwd_dkdv_hash_train_T16384_traffic.txt")
# files that determine the code of the attention kernels and the tile lists they walk
KERNEL_SOURCES = ["attn_bwd.hip", "attn_fwd.hip", "meta.hip", "scfa_pipe.hpp", "scfa_device.hpp",
                  "scfa_internal.hpp", "../build.py"]


def kernel_source_digest():
    h = hashlib.sha256()
    base = os.path.join(ROOT, "sparse_causal_attention_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.normpath(os.path.join(base, name)), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(tile_rule, view, backward):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None
    (None too when the summary was taken with the other tile rule, the other view of the rows or the
    other backward)."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith((" ", "#")))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if (kv.get("source_digest") != kernel_source_digest() or kv.get("tile_rule") != tile_rule
            or kv.get("rows") != view or kv.get("backward", "recompute") != backward):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_inputs(w, torch):
    import numpy as np

    from gen import head_inputs, lsh_rotation

    heads = [[head_inputs(w, b, h) for h in range(w.H)] for b in range(w.B)]

    def st(f):
        return np.stack([np.stack([f(x) for x in row]) for row in heads])

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    # Q and K share one allocation, Q first: [2B, H, T, d].  R is per head and shared by the batch, so one
    # LSH + sort call over the stacked tensor hashes and orders both (batch entries B.. are K's).
    qk = to(np.concatenate([st(lambda x: x.q), st(lambda x: x.k)]))
    q, k = qk[: w.B], qk[w.B:]
    v, do = to(st(lambda x: x.v)), to(st(lambda x: x.do))
    R = torch.from_numpy(np.stack([lsh_rotation(w, h) for h in range(w.H)])).to(dev)
    return q, k, v, do, R, qk


def tile_work(meta, Tq, Tk, block, torch):
    """Sum over executed tiles of bq*bk (real extents), from the row lists."""
    cnt = meta["row_count"].long()  # [B,H,nq]
    lst = meta["row_list"].long() & 0x7FFFFFFF  # [B,H,nq,nk]
    nq, nk = lst.shape[2], lst.shape[3]
    valid = torch.arange(nk, device=lst.device)[None, None, None, :] < cnt[..., None]
    bq = torch.clamp(Tq - torch.arange(nq, device=lst.device) * block, max=block)  # [nq]
    bk_all = torch.clamp(Tk - torch.arange(nk, device=lst.device) * block, max=block)  # [nk]
    bk = bk_all[lst.clamp(max=nk - 1)] * valid
    return int((bk.sum(-1) * bq[None, None, :]).sum().item()), int(cnt.sum().item())


class Timer:
    """HIP events between the calls of one step (torch's current stream, which the library uses).

    ``only`` (names) restricts the events to the boundaries of those calls: events between all calls of the
    16k step cost about 4 % of its time, two events around one call about 1 %."""

    def __init__(self, torch, names, only=None):
        self.torch = torch
        self.names = names
        self.only = set(names if only is None else only)
        self.samples = {n: [] for n in names}
        self.pending = []
        self.i = 0

    def _boundary(self):
        # boundary i ends call i - 1 and starts call i
        i = self.i
        if (i < len(self.names) and self.names[i] in self.only) or (0 < i <= len(self.names) and
                                                                     self.names[i - 1] in self.only):
            ev = self.torch.cuda.Event(enable_timing=True)
            ev.record()
            self.pending[-1][i] = ev

    def begin(self):
        self.i = 0
        self.pending.append({})
        self._boundary()

    def mark(self):
        self.i += 1
        self._boundary()

    def collect(self):
        for evs in self.pending:
            for j, n in enumerate(self.names):
                if j in evs and j + 1 in evs:
                    self.samples[n].append(evs[j].elapsed_time(evs[j + 1]))
        self.pending = []

    def median_ms(self, n):
        s = sorted(self.samples[n])
        if not s:
            return float("nan")
        m = len(s) // 2
        return s[m] if len(s) % 2 else 0.5 * (s[m - 1] + s[m])

    def step_median_ms(self):
        """Median over steps of the event time from the first call's start to the last call's end."""
        tot = sorted(sum(self.samples[n][i] for n in self.names) for i in range(len(self.samples[self.names[0]])))
        if not tot:
            return float("nan")
        m = len(tot) // 2
        return tot[m] if len(tot) % 2 else 0.5 * (tot[m - 1] + tot[m])


def run_step(scfa, w, q, k, v, do, R, timer=None, exact=True, copy_sorted=False, qk=None, ds=None,
             orig_rows=True):
    """One step.  By default the sorts return only bucket ids, positions and the permutations, and
    the attention kernels read Q, dO, K and V through the permutations (row indirection); with
    copy_sorted the sorts also copy the rows into sorted order and attention reads the copies.
    Outputs (O, lse, dQ, dK, dV) are in sorted order either way, bit-identical.  The returned
    metadata dict also holds the sort results (bucket ids, positions and, for the permuted view,
    the permutations).

    With qk (Q and K stacked in one [2B, H, T, d] allocation, q and k its halves) and rows read
    through the permutations, one LSH + sort call serves both tensors.

    With ds (a dS buffer, see prepare_ds) the backward stores every live tile's dS in the dK/dV
    kernel and computes dQ from the stored tiles (tile slots built with the lists, then the
    preprocess for D, dK/dV, dQ); without it the dQ kernel recomputes S, P and dP.

    With orig_rows (the default) and rows read through the permutations, the kernels write O, lse,
    dQ, dK and dV at the caller's rows (token order) directly: no separate un-sort."""
    nb, blk, sc = w.n_buckets, w.block, w.scale
    B = q.shape[0]
    if timer:
        timer.begin()
    if copy_sorted:
        qh, qi, _, qs, dos = scfa.lsh_bucket_sort(q, R, nb, companion=do)
        if timer:
            timer.mark()
        kh, ki, _, ks, vs = scfa.lsh_bucket_sort(k, R, nb, companion=v)
        rows = {}
    elif qk is not None:
        hh, ii, pp, _, _ = scfa.lsh_bucket_sort(qk, R, nb, want_x=False)
        qh, kh, qi, ki, qp, kp = hh[:B], hh[B:], ii[:B], ii[B:], pp[:B], pp[B:]
        qs, dos, ks, vs = q, do, k, v
        rows = {"q_rows": qp, "k_rows": kp}
    else:
        qh, qi, qp, _, _ = scfa.lsh_bucket_sort(q, R, nb, want_x=False)
        if timer:
            timer.mark()
        kh, ki, kp, _, _ = scfa.lsh_bucket_sort(k, R, nb, want_x=False)
        qs, dos, ks, vs = q, do, k, v
        rows = {"q_rows": qp, "k_rows": kp}
    if timer:
        timer.mark()
    meta = scfa.block_meta(qi, ki, qh, kh, block=blk, with_cols=True, exact=exact)
    if ds is not None:
        scfa.tile_slots(meta)
    if timer:
        timer.mark()
    meta.update(q_hash=qh, q_idx=qi, k_hash=kh, k_idx=ki, **({"q_perm": rows["q_rows"], "k_perm": rows["k_rows"]}
                                                             if rows else {}))
    fl = scfa.FLAG_ORIG_ROWS if (orig_rows and rows) else 0
    meta["outputs"] = "caller rows" if fl else "view rows"
    o, lse = scfa.attn_fwd_lists(qs, ks, vs, qi, ki, qh, kh, meta, block=blk, scale=sc, flags=fl, **rows)
    if timer:
        timer.mark()
    if ds is None:
        dq, delta = scfa.attn_bwd_dq_lists(qs, ks, vs, o, lse, dos, qi, ki, qh, kh, meta, block=blk, scale=sc,
                                           flags=fl, **rows)
        if timer:
            timer.mark()
        dk, dv = scfa.attn_bwd_dkdv_lists(qs, ks, vs, lse, dos, delta, qi, ki, qh, kh, meta, block=blk, scale=sc,
                                          flags=fl, **rows)
        if timer:
            timer.mark()
    else:
        delta = scfa.attn_bwd_prep(o, lse, dos, q_rows=rows.get("q_rows"), flags=fl)
        if timer:
            timer.mark()
        dk, dv = scfa.attn_bwd_dkdv_ds_lists(qs, ks, vs, lse, dos, delta, qi, ki, qh, kh, meta, ds, block=blk,
                                             scale=sc, flags=fl, **rows)
        if timer:
            timer.mark()
        dq = scfa.attn_bwd_dq_ds_lists(qs, ks, vs, o, lse, dos, qi, ki, qh, kh, meta, ds, delta, block=blk,
                                       scale=sc, flags=fl, **rows)
        if timer:
            timer.mark()
    return meta, (o, lse, dq, dk, dv)


def prepare_ds(scfa, torch, w, q, k, R, qk=None, exact=True, copy_sorted=False):
    """A dS buffer holding every live tile of the step's inputs (sized once, before timing, from one
    metadata pass, as a caller sizes any workspace)."""
    B = q.shape[0]
    if qk is not None and not copy_sorted:
        hh, ii, _, _, _ = scfa.lsh_bucket_sort(qk, R, w.n_buckets, want_x=False)
        qh, kh, qi, ki = hh[:B], hh[B:], ii[:B], ii[B:]
    else:
        qh, qi, _, _, _ = scfa.lsh_bucket_sort(q, R, w.n_buckets, want_x=False)
        kh, ki, _, _, _ = scfa.lsh_bucket_sort(k, R, w.n_buckets, want_x=False)
    meta = scfa.block_meta(qi, ki, qh, kh, block=w.block, with_cols=True, exact=exact)
    total = int(meta["col_count"].sum().item())
    return scfa.ds_buffer(total, w.block, device=q.device)


STEP_CALLS = ["lsh_sort_qk", "block_meta", "fwd", "bwd_dq", "bwd_dkdv"]
STEP_CALLS_COPIED = ["lsh_sort_q", "lsh_sort_k", "block_meta", "fwd", "bwd_dq", "bwd_dkdv"]
STEP_CALLS_DS = ["lsh_sort_qk", "block_meta", "fwd", "bwd_prep", "bwd_dkdv", "bwd_dq"]
STEP_CALLS_COPIED_DS = ["lsh_sort_q", "lsh_sort_k", "block_meta", "fwd", "bwd_prep", "bwd_dkdv", "bwd_dq"]


def step_calls(copy_sorted, stored_ds=False):
    if stored_ds:
        return STEP_CALLS_COPIED_DS if copy_sorted else STEP_CALLS_DS
    return STEP_CALLS_COPIED if copy_sorted else STEP_CALLS


def run_dense(scfa, w, q, k, v, do, timer=None):
    blk, sc = w.block, w.scale
    if timer:
        timer.begin()
    o, lse = scfa.attn_fwd_lists(q, k, v, None, None, None, None, None, block=blk, scale=sc)
    if timer:
        timer.mark()
    dq, delta = scfa.attn_bwd_dq_lists(q, k, v, o, lse, do, None, None, None, None, None, block=blk, scale=sc)
    if timer:
        timer.mark()
    scfa.attn_bwd_dkdv_lists(q, k, v, lse, do, delta, None, None, None, None, None, block=blk, scale=sc)
    if timer:
        timer.mark()


DENSE_CALLS = ["dense_fwd", "dense_bwd_dq", "dense_bwd_dkdv"]


CPU_SAMPLE_S = 10.0  # the CPU oracle runs heads until at least this much work has been timed


def cpu_baseline(w, tile_units_per_head):
    """The fp64 oracle on heads (b=0, h=0, 1, ...) of the workload (LSH, sort, masked attention fwd + bwd),
    until at least CPU_SAMPLE_S seconds of work; each head is credited with the workload's average
    executed-tile flops per head."""
    import numpy as np

    from gen import head_inputs, lsh_rotation
    from oracle import attention as A
    from oracle import lsh

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    dt, heads = 0.0, 0
    while heads < w.H and (heads == 0 or dt < CPU_SAMPLE_S):
        hi = head_inputs(w, 0, heads)  # inputs are drawn outside the timed work
        R = lsh_rotation(w, heads)
        t0 = time.perf_counter()
        bq, bk = lsh.buckets(hi.q, R), lsh.buckets(hi.k, R)
        pq, hq, iq = lsh.bucket_sort(bq, hi.q_pos)
        pk, hk, ik = lsh.bucket_sort(bk, hi.k_pos)
        A.forward(hi.q[pq], hi.k[pk], hi.v[pk], iq, ik, hq, hk, w.scale)
        A.backward(hi.q[pq], hi.k[pk], hi.v[pk], hi.do[pq], iq, ik, hq, hk, w.scale)
        dt += time.perf_counter() - t0
        heads += 1
    flops = 14.0 * tile_units_per_head * w.d * heads
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} heads (b=0, h=0..{heads - 1}) of the workload, run until at least {CPU_SAMPLE_S:.0f} s of "
                  f"work: LSH + sort of Q and K, dense masked fp64 forward and backward over {w.T} tokens each; "
                  f"{dt:.2f} s, credited with the workload's average executed-tile flops per head",
        "seconds": dt,
        "heads": heads,
    }


def _time_steps(torch, fn, steps, warmup, timer=None):
    _warm(torch, fn, warmup, SETTLE_MS)
    t0 = time.perf_counter()
    out = None
    for _ in range(steps):
        out = fn(timer)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3, out


# Block sizes the library's kernels take.  The dense-causal comparator is timed at each and the faster one is
# kept, so a speedup is never quoted against a slower configuration of the same library.
DENSE_BLOCKS = (64, 128)
# Clocks settle after a few tens of milliseconds of work (measured: the first 20 steps after a short warmup
# run about 12 % slower than the steady state reached after about 40 steps of the 16k training step).
SETTLE_MS = 50.0


def time_with_breakdown(torch, fn, calls, steps, warmup, timed_only=()):
    """Warm-up, a breakdown pass of `steps` steps with HIP events between all calls, then the timed `steps`
    steps with events only around the calls in `timed_only`.  Returns (ms per timed step, the last timed
    step's result, breakdown Timer, timed Timer)."""
    _warm(torch, fn, warmup, SETTLE_MS)
    breakdown = Timer(torch, calls)
    for _ in range(steps):
        fn(breakdown)
    torch.cuda.synchronize()
    breakdown.collect()
    timed = Timer(torch, calls, only=timed_only)
    t0 = time.perf_counter()  # the breakdown pass ended synchronised
    out = None
    for _ in range(steps):
        out = fn(timed)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    timed.collect()
    return ms, out, breakdown, timed


def _warm(torch, fn, n, min_ms=0.0):
    """n untimed calls of fn(None), then more until min_ms of wall time has passed; returns the count."""
    t0 = time.perf_counter()
    done = 0
    while done < n or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn(None)
        done += 1
        if done >= n:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return done


def time_dense(torch, run, blocks, steps, warmup, timer_names=None):
    """The dense-causal comparator, run(block, timer) being one step, at each block size in blocks.
    Returns (fastest ms per step, its block, {block: ms per step}, a Timer over the fastest block's calls
    when timer_names is given, else None)."""
    by_block = {}
    for b in blocks:
        for _ in range(warmup):
            run(b, None)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            run(b, None)
        torch.cuda.synchronize()
        by_block[b] = (time.perf_counter() - t1) / steps * 1e3
    best = min(by_block, key=by_block.get)
    timer = None
    if timer_names:
        timer = Timer(torch, timer_names)
        for _ in range(steps):
            run(best, timer)
        torch.cuda.synchronize()
        timer.collect()
    return by_block[best], best, {b: round(t, 4) for b, t in by_block.items()}, timer


def _gpu_normal(torch, shape, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)


def _dense_step(scfa, q, k, v, do, block=64):
    o, lse = scfa.qk_sparse_fwd(q, k, v, block=block)
    scfa.qk_sparse_bwd(q, k, v, o, lse, do, block=block)


def sweep_drop(scfa, torch, rates, args):
    """QK-sparse training step against the naive ways of dropping tokens, at each drop rate.

    * scfa: compaction of Q, K, V, dO to the kept tokens, QK-sparse forward + backward (tile pruning on the
      kept positions), outputs put back at the original positions;
    * naive_compacted: the same compacted tensors, but every tile computed and then masked
      (NO_PRUNE + FORCE_MASK): dropping without SCFA's tile rules;
    * naive_full_masked: full-length causal attention with the dropped tokens masked out (a dropped query
      carries position -1 and admits no key, a dropped key position 2^31 - 1 and no query admits it): the
      dropped tokens still occupy the tiles;
    * dense_causal: full-length causal attention, nothing dropped.
    """
    B, H, T, d = 4, 12, 8192, 64
    q, k, v, do = (_gpu_normal(torch, (B, H, T, d), 100 + i) for i in range(4))
    dense_ms, dense_blk, _, _ = time_dense(torch, lambda b, _: _dense_step(scfa, q, k, v, do, b), DENSE_BLOCKS,
                                           max(3, args.steps // 2), max(1, min(args.warmup, 3)))
    naive_flags = scfa.FLAG_NO_PRUNE | scfa.FLAG_FORCE_MASK
    pos = torch.arange(T, device="cuda:0", dtype=torch.int32).expand(B, H, T)
    for rate in rates:
        n_keep = max(1, int(round((1.0 - rate) * T)))
        g = torch.Generator(device="cuda:0")
        g.manual_seed(7)
        keep = torch.stack([torch.stack([torch.sort(torch.randperm(T, generator=g, device="cuda:0")[:n_keep])[0]
                                         for _ in range(H)]) for _ in range(B)]).to(torch.int32).contiguous()
        kept = torch.zeros((B, H, T), dtype=torch.bool, device="cuda:0")
        kept.scatter_(2, keep.long(), True)
        q_pos = torch.where(kept, pos, torch.full_like(pos, -1)).contiguous()
        k_pos = torch.where(kept, pos, torch.full_like(pos, 2**31 - 1)).contiguous()

        def compacted(flags):
            def step(_):
                qc, kc, vc, gc = (scfa.gather_rows(x, keep) for x in (q, k, v, do))
                o, lse = scfa.qk_sparse_fwd(qc, kc, vc, keep, keep, flags=flags)
                grads = scfa.qk_sparse_bwd(qc, kc, vc, o, lse, gc, keep, keep, flags=flags)
                for x in (o, *grads):
                    scfa.scatter_rows(x, keep, T)
            return step

        def full_masked(_):
            o, lse = scfa.qk_sparse_fwd(q, k, v, q_pos, k_pos)
            scfa.qk_sparse_bwd(q, k, v, o, lse, do, q_pos, k_pos)

        ms, _ = _time_steps(torch, compacted(0), args.steps, args.warmup)
        naive_c_ms, _ = _time_steps(torch, compacted(naive_flags), max(3, args.steps // 2), 1)
        naive_f_ms, _ = _time_steps(torch, full_masked, max(3, args.steps // 2), 1)
        print(json.dumps({"sweep": "qk_drop_rate", "B": B, "H": H, "T": T, "d": d, "drop_rate": rate,
                          "kept": n_keep, "scfa_step_ms": round(ms, 4),
                          "naive_compacted_ms": round(naive_c_ms, 4),
                          "naive_full_masked_ms": round(naive_f_ms, 4), "dense_causal_ms": round(dense_ms, 4),
                          "dense_causal_block": dense_blk,
                          "speedup_vs_naive_compacted": round(naive_c_ms / ms, 3),
                          "speedup_vs_naive_full_masked": round(naive_f_ms / ms, 3),
                          "speedup_vs_dense_causal": round(dense_ms / ms, 3),
                          "naive_compacted_vs_dense_causal": round(dense_ms / naive_c_ms, 3),
                          "scfa_step": "gather Q,K,V,dO + QK-sparse fwd + bwd + scatter O,dQ,dK,dV",
                          "naive_compacted": "same, every tile computed then masked (NO_PRUNE + FORCE_MASK)",
                          "naive_full_masked": "full-length causal fwd + bwd, dropped tokens masked by position"}),
              flush=True)


def sweep_length(scfa, torch, lengths, args):
    B, H, d, nb = 1, 8, 64, 32
    g = torch.Generator(device="cuda:0")
    g.manual_seed(3)
    R = torch.randn((H, d, nb // 2), generator=g, device="cuda:0", dtype=torch.float32)
    naive_flags = scfa.FLAG_NO_PRUNE | scfa.FLAG_FORCE_MASK
    for T in lengths:
        q, k, v, do = (_gpu_normal(torch, (B, H, T, d), 200 + i) for i in range(4))
        train = T <= 32768
        state = {}

        def scfa_step(_):
            qh, qi, _, qs, dos = scfa.lsh_bucket_sort(q, R, nb, companion=do)
            kh, ki, _, ks, vs = scfa.lsh_bucket_sort(k, R, nb, companion=v)
            o, lse = scfa.hash_sparse_fwd(qs, ks, vs, qi, ki, qh, kh)
            if train:
                scfa.hash_sparse_bwd(qs, ks, vs, o, lse, dos, qi, ki, qh, kh)
            state["sorted"] = (qs, ks, vs, dos, qi, ki, qh, kh, o, lse)

        steps = args.steps if T <= 262144 else max(2, args.steps // 4)
        ms, _ = _time_steps(torch, scfa_step, steps, min(args.warmup, 2))
        line = {"sweep": "hash_length", "B": B, "H": H, "T": T, "d": d, "n_buckets": nb,
                "pass": "fwd+bwd" if train else "fwd", "scfa_ms": round(ms, 4)}
        if train:
            qs, ks, vs, dos, qi, ki, qh, kh, o, lse = state["sorted"]

            def naive(_):
                o2, l2 = scfa.hash_sparse_fwd(qs, ks, vs, qi, ki, qh, kh, flags=naive_flags)
                scfa.hash_sparse_bwd(qs, ks, vs, o2, l2, dos, qi, ki, qh, kh, flags=naive_flags)

            nd = max(2, args.steps // 4)
            naive_ms, _ = _time_steps(torch, naive, nd, 1)
            dense_ms, dense_blk, _, _ = time_dense(torch, lambda b, _: _dense_step(scfa, q, k, v, do, b),
                                                   DENSE_BLOCKS, nd, 1)
            line.update({"naive_hash_ms": round(naive_ms, 4), "dense_causal_ms": round(dense_ms, 4),
                         "dense_causal_block": dense_blk,
                         "speedup_vs_dense_causal": round(dense_ms / ms, 3),
                         "speedup_vs_naive_hash": round(naive_ms / ms, 3)})
        print(json.dumps(line), flush=True)
        del q, k, v, do, state
        torch.cuda.empty_cache()


def sweep_ragged(scfa, torch, args):
    """QK-sparse training over heads with their own kept counts: packed heads against the padded layout.

    Each of the B*H heads drops its own share of tokens (drop rate drawn per head), so kept counts differ.
    * packed: the heads back to back with no padding, per-head offsets (block_meta_varlen + the varlen
      forward, dQ and dK/dV calls);
    * padded: every head padded to the longest kept count, padding queries at position -1 and padding keys at
      2^31 - 1 (block_meta + the list forward, dQ and dK/dV calls).
    Both time metadata + forward + backward with the compacted tensors already resident; the outputs agree
    bit for bit on the real rows.
    """
    import numpy as np

    B, H, T, d, block = 4, 12, 8192, 64, 64
    for name, lo, hi in (("uniform drop 10-90%", 0.1, 0.9), ("skewed: drop 90% except one head per batch", 0.9, 0.9)):
        rng = np.random.default_rng(11)
        rates = rng.uniform(lo, hi, B * H)
        if lo == hi:
            rates[::H] = 0.0
        kept = [max(1, int(round((1.0 - r) * T))) for r in rates]
        pos = [np.sort(rng.choice(T, n, replace=False)).astype(np.int32) for n in kept]
        off = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
        total, mx = int(off[-1]), max(kept)
        q, k, v, do = (_gpu_normal(torch, (total, d), 300 + i) for i in range(4))
        idx = torch.from_numpy(np.concatenate(pos)).cuda()
        offs = torch.from_numpy(off).cuda()
        pq = np.full((B * H, mx), -1, np.int32)
        pk = np.full((B * H, mx), 2**31 - 1, np.int32)
        rows = np.full((B * H, mx), -1, np.int64)
        for i, p in enumerate(pos):
            pq[i, :len(p)] = p
            pk[i, :len(p)] = p
            rows[i, :len(p)] = np.arange(off[i], off[i + 1])
        pqi, pki = (torch.from_numpy(a.reshape(B, H, mx)).cuda() for a in (pq, pk))
        sel = torch.from_numpy(rows.reshape(-1)).cuda()
        have = sel >= 0

        def padded_of(x):
            y = torch.zeros((B * H * mx, d), dtype=x.dtype, device=x.device)
            y[have] = x[sel[have]]
            return y.view(B, H, mx, d)

        Pq, Pk, Pv, Pdo = (padded_of(x) for x in (q, k, v, do))
        mt = dict(H=H, max_Tq=mx, max_Tk=mx, block=block)

        def marked(t):
            if t:
                t.mark()

        def packed(t):
            if t:
                t.begin()
            meta = scfa.block_meta_varlen(offs, offs, idx, idx, **mt)
            marked(t)
            o, lse = scfa.attn_fwd_varlen(q, k, v, offs, offs, idx, idx, None, None, meta, **mt)
            marked(t)
            dq, delta = scfa.attn_bwd_dq_varlen(q, k, v, o, lse, do, offs, offs, idx, idx, None, None, meta, **mt)
            marked(t)
            scfa.attn_bwd_dkdv_varlen(q, k, v, lse, do, delta, offs, offs, idx, idx, None, None, meta, **mt)
            marked(t)
            return o

        def padded(t):
            if t:
                t.begin()
            meta = scfa.block_meta(pqi, pki, block=block, with_cols=True, exact=True)
            marked(t)
            o, lse = scfa.attn_fwd_lists(Pq, Pk, Pv, pqi, pki, None, None, meta, block=block)
            marked(t)
            dq, delta = scfa.attn_bwd_dq_lists(Pq, Pk, Pv, o, lse, Pdo, pqi, pki, None, None, meta, block=block)
            marked(t)
            scfa.attn_bwd_dkdv_lists(Pq, Pk, Pv, lse, Pdo, delta, pqi, pki, None, None, meta, block=block)
            marked(t)
            return o

        calls = ["block_meta", "fwd", "bwd_dq", "bwd_dkdv"]
        t_packed, t_padded = Timer(torch, calls), Timer(torch, calls)
        ms_packed, o1 = _time_steps(torch, packed, args.steps, args.warmup, t_packed)
        ms_padded, o2 = _time_steps(torch, padded, args.steps, args.warmup, t_padded)
        t_packed.collect()
        t_padded.collect()
        same = bool(torch.equal(o1[sel[have]], o2.reshape(-1, d)[have]))
        print(json.dumps({"sweep": "ragged_heads", "heads": name, "B": B, "H": H, "T": T, "d": d, "block": block,
                          "kept_min": min(kept), "kept_max": mx, "rows_packed": total, "rows_padded": B * H * mx,
                          "packed_ms": round(ms_packed, 4), "padded_ms": round(ms_padded, 4),
                          "speedup_packed_vs_padded": round(ms_padded / ms_packed, 3),
                          "qkvdo_bytes_packed": 4 * total * d * 2, "qkvdo_bytes_padded": 4 * B * H * mx * d * 2,
                          "outputs_equal": same,
                          "packed_per_call_ms": {n: round(t_packed.median_ms(n), 4) for n in calls},
                          "padded_per_call_ms": {n: round(t_padded.median_ms(n), 4) for n in calls},
                          "per_call_stat": f"median of {args.steps} HIP-event samples per call",
                          "step": "block lists + QK-sparse fwd + dQ + dK/dV (compacted tensors resident)"}),
              flush=True)
        del q, k, v, do, Pq, Pk, Pv, Pdo
        torch.cuda.empty_cache()


def measure_rows(scfa, torch, w, q, k, v, do, R, args):
    """HBM throughput of gather_rows / scatter_rows at the step's shape."""
    import numpy as np

    qh, qi, qperm, qs, dos = scfa.lsh_bucket_sort(q, R, w.n_buckets, companion=do)
    rows_out = [qs, dos, qs, dos]  # four [B,H,T,d] tensors, as O, dQ, dK, dV
    perm = qperm
    n_keep = int(round(0.7 * w.T))
    rng = np.random.default_rng(0)
    keep = torch.from_numpy(np.stack([np.stack([np.sort(rng.choice(w.T, n_keep, replace=False)).astype(np.int32)
                                                for _ in range(w.H)]) for _ in range(w.B)])).to(q.device)
    row_bytes = w.d * 2

    def unsort(_):
        for x in rows_out:
            scfa.scatter_rows(x, perm, w.T, zero_fill=False)

    def compact(_):
        for x in (q, k, v):
            scfa.gather_rows(x, keep)

    ms_u, _ = _time_steps(torch, unsort, args.steps, args.warmup)
    ms_c, _ = _time_steps(torch, compact, args.steps, args.warmup)
    bytes_u = 4 * (w.B * w.H * w.T) * (2 * row_bytes + 4)  # read row + index, write row
    bytes_c = 3 * (w.B * w.H * n_keep) * (2 * row_bytes + 4)
    print(json.dumps({
        "measure": "row gather / scatter", "workload": w.name,
        "unsort_4_tensors_ms": round(ms_u, 4), "unsort_GBps": round(bytes_u / (ms_u * 1e-3) / 1e9, 1),
        "compact_3_tensors_ms": round(ms_c, 4), "compact_GBps": round(bytes_c / (ms_c * 1e-3) / 1e9, 1),
        "peak_GBps": PEAK_HBM_GBS, "kept_fraction": 0.7,
        "bytes_per_row": "row read + row written + 4-byte index",
    }), flush=True)


def sweep_buckets(scfa, torch, w, q, k, v, do, qk, nbs, args):
    """Same shape and inputs, LSH rotations drawn per bucket count (seeded by the workload)."""
    import dataclasses

    import numpy as np

    from gen import lsh_rotation

    dense_ms, dense_blk, _, _ = time_dense(
        torch, lambda b, t: run_dense(scfa, dataclasses.replace(w, block=b), q, k, v, do, t), DENSE_BLOCKS,
        max(3, args.steps // 2), max(1, min(args.warmup, 3)))
    for nb in nbs:
        wn = dataclasses.replace(w, n_buckets=nb, name=f"{w.name.rsplit('_nb', 1)[0]}_nb{nb}")
        R = torch.from_numpy(np.stack([lsh_rotation(wn, h) for h in range(w.H)])).to("cuda:0")
        ds = prepare_ds(scfa, torch, wn, q, k, R, qk, not args.range_lists, args.copy_sorted) if args.stored_ds \
            else None
        calls = step_calls(args.copy_sorted, ds is not None)
        ms, (meta, _), timer, _ = time_with_breakdown(
            torch, lambda t: run_step(scfa, wn, q, k, v, do, R, t, not args.range_lists, args.copy_sorted, qk, ds),
            calls, args.steps, args.warmup)
        units, tiles = tile_work(meta, w.Tq, w.Tk, w.block, torch)
        per_call = {n: round(timer.median_ms(n), 4) for n in calls}
        attn_ms = sum(t for n, t in per_call.items() if not n.startswith("lsh"))
        del ds
        nq = (w.T + w.block - 1) // w.block
        print(json.dumps({
            "sweep": "n_buckets", "workload": wn.name, "n_buckets": nb, "executed_tiles": tiles,
            "mean_live_kblocks_per_qblock": round(tiles / (w.B * w.H * nq), 2),
            "ms_per_step": round(ms, 4), "tflops": round(14.0 * units * w.d / (ms * 1e-3) / 1e12, 2),
            "dense_causal_ms": round(dense_ms, 4), "dense_causal_block": dense_blk,
            "speedup_vs_dense_causal": round(dense_ms / ms, 3),
            "speedup_vs_dense_causal_excl_lsh": round(dense_ms / attn_ms, 3), "per_call_ms": per_call,
        }), flush=True)


# ---------------------------------------------------------------------------
# The other workloads (--workload 2, 3, 5): one JSON line each, same metric.
# ---------------------------------------------------------------------------
def _median(xs):
    xs = sorted(xs)
    m = len(xs) // 2
    return xs[m] if len(xs) % 2 else 0.5 * (xs[m - 1] + xs[m])


def _full_length_inputs(w, torch, names, seed):
    """Full-length [B,H,T,d] bf16 tensors drawn on the GPU (seeded) and the workload's kept positions
    [B,H,n_keep] (gen.keep_set, shared by Q and K)."""
    import numpy as np

    from gen import keep_set

    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    full = [torch.randn((w.B, w.H, w.T, w.d), generator=g, device="cuda:0", dtype=torch.float32).to(torch.bfloat16)
            for _ in names]
    keep = torch.from_numpy(np.stack([np.stack([keep_set(w, b, h)[0] for h in range(w.H)])
                                      for b in range(w.B)])).to("cuda:0")
    return dict(zip(names, full)), keep


def time_graph(torch, step, steps):
    """ms per step with the whole step captured once as a HIP graph and replayed (the host enqueues one graph
    launch per step instead of every kernel).  The step is warmed up on the capture stream first."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            step(None)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    _warm(torch, lambda _: g.replay(), 3, SETTLE_MS)
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def _dropped(keep, T, torch):
    """The positions [B,H,T - n] (ascending) that the kept set [B,H,n] leaves out, per head."""
    B, H, n = keep.shape
    mask = torch.ones((B, H, T), dtype=torch.bool, device=keep.device)
    mask.scatter_(2, keep.long(), False)
    pos = torch.arange(T, dtype=torch.int32, device=keep.device).expand(B, H, T)
    return pos[mask].view(B, H, T - n).contiguous()


def _roofline(kernel, flops, ms):
    achieved = flops / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "avg_launch_ms": ms, "algorithmic_flops_per_launch": flops}


def workload_setup(scfa, torch, wid):
    """Inputs of workload 2, 3 or 5 resident in HBM, and its step (see bench_workload).

    Returns (w, step, calls, dense_in): step(timer) runs one step (marking the timer after each call
    in ``calls`` when one is given) and returns (meta, outputs); dense_in are the full-length (q, k, v,
    dout) the dense-causal comparator reads."""
    import numpy as np

    from gen import WORKLOADS, head_inputs, lsh_rotation

    w = WORKLOADS[wid]
    blk, sc = w.block, w.scale
    dev = torch.device("cuda:0")
    _log(f"[bench] workload {w.name}: inputs")
    R = None
    if w.n_buckets:
        R = torch.from_numpy(np.stack([lsh_rotation(w, h) for h in range(w.H)])).to(dev)
    if wid == 2:
        heads = [[head_inputs(w, b, h) for h in range(w.H)] for b in range(w.B)]
        st = lambda f: np.stack([np.stack([f(x) for x in row]) for row in heads])  # noqa: E731
        to = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
        qk = to(np.concatenate([st(lambda x: x.q), st(lambda x: x.k)]))
        q, k = qk[: w.B], qk[w.B:]
        v = to(st(lambda x: x.v))
        dense_in = (q, k, v, None)
        calls = ["lsh_sort_qk", "block_meta", "fwd"]

        def step(t):
            if t:
                t.begin()
            hh, ii, pp, _, _ = scfa.lsh_bucket_sort(qk, R, w.n_buckets, want_x=False)
            B = w.B
            qh, kh, qi, ki = hh[:B], hh[B:], ii[:B], ii[B:]
            if t:
                t.mark()
            meta = scfa.block_meta(qi, ki, qh, kh, block=blk, with_cols=False, exact=True)
            if t:
                t.mark()
            o, lse = scfa.attn_fwd_lists(q, k, v, qi, ki, qh, kh, meta, block=blk, scale=sc, q_rows=pp[:B],
                                         k_rows=pp[B:])
            if t:
                t.mark()
            return meta, dict(o=o, lse=lse, hash=hh, idx=ii, perm=pp)
    elif wid == 3:
        full, keep = _full_length_inputs(w, torch, ("q", "k", "v", "do"), 300 + wid)
        drop = _dropped(keep, w.T, torch)
        q, k, v, do = (full[n] for n in ("q", "k", "v", "do"))
        dense_in = (q, k, v, do)
        calls = ["block_meta", "fwd", "bwd_dq", "bwd_dkdv", "clear_dropped"]
        rows = dict(q_rows=keep, k_rows=keep, flags=scfa.FLAG_ORIG_ROWS, block=blk, scale=sc)

        def step(t):
            if t:
                t.begin()
            meta = scfa.block_meta(keep, keep, block=blk, with_cols=True, exact=True)
            if t:
                t.mark()
            o, lse = scfa.attn_fwd_lists(q, k, v, keep, keep, None, None, meta, **rows)
            if t:
                t.mark()
            dq, delta = scfa.attn_bwd_dq_lists(q, k, v, o, lse, do, keep, keep, None, None, meta, **rows)
            if t:
                t.mark()
            dk, dv = scfa.attn_bwd_dkdv_lists(q, k, v, lse, do, delta, keep, keep, None, None, meta, **rows)
            if t:
                t.mark()
            for x in (o, dq, dk, dv):
                scfa.zero_rows(x, drop)
            if t:
                t.mark()
            return meta, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    elif wid == 5:
        full, keep = _full_length_inputs(w, torch, ("q", "k", "v"), 300 + wid)
        B = w.B
        qk = torch.cat([full.pop("q"), full.pop("k")])  # [2B,H,T,d]: Q and K stacked along the batch
        v = full["v"]
        dense_in = (qk[:B], qk[B:], v, None)
        keep2 = torch.cat([keep, keep]).contiguous()
        drop = _dropped(keep, w.T, torch)
        calls = ["lsh_sort_qk", "block_meta", "fwd", "clear_dropped"]

        def step(t):
            if t:
                t.begin()
            hh, ii, _, _, _ = scfa.lsh_bucket_sort(qk, R, w.n_buckets, idx=keep2, idx_ascending=True, want_x=False,
                                                   x_rows=keep2)
            qh, kh, qi, ki = hh[:B], hh[B:], ii[:B], ii[B:]
            if t:
                t.mark()
            meta = scfa.block_meta(qi, ki, qh, kh, block=blk, with_cols=False, exact=True)
            if t:
                t.mark()
            # sorted view row i is the token at original position qi[i]: read and write that row
            o, lse = scfa.attn_fwd_lists(qk[:B], qk[B:], v, qi, ki, qh, kh, meta, block=blk, scale=sc, q_rows=qi,
                                         k_rows=ki, flags=scfa.FLAG_ORIG_ROWS)
            if t:
                t.mark()
            scfa.zero_rows(o, drop)
            if t:
                t.mark()
            return meta, dict(o=o, lse=lse, hash=hh, idx=ii)
    else:
        raise SystemExit(f"--workload {wid}: choose 2, 3, 5 (4 is the default benchmark line)")
    return w, step, calls, dense_in



def bench_workload(scfa, torch, wid, args):
    """One benchmark line for workload 2 (Hash-sparse forward, 8k tokens), 3 (QK-sparse training step with
    30 % of the tokens dropped, 8k tokens) or 5 (50 % drop, then Hash-sparse forward, 1M tokens).  The step
    runs every row of the hot path the workload has, from inputs resident in HBM:
      2: LSH + sort of Q and K (one call over both), block lists, forward over the sorted view;
      3: block lists, forward, dQ, dK/dV over the kept rows of the full-length Q, K, V, dO (read in place
         at the kept positions, outputs written there), and the dropped positions' output rows cleared;
      5: LSH + sort of the kept rows of the full-length Q and K (one call, rows read in place), block lists,
         the forward reading Q, K, V at the kept positions and writing O there, and the dropped rows of O
         cleared.
    No kept row is copied into a compact tensor: positions double as row indices into the inputs.
    The dense-causal comparator is the same library's dense mode on the original [B,H,T,d] tensors."""
    w, step, calls, dense_in = workload_setup(scfa, torch, wid)
    blk, sc = w.block, w.scale
    steps = args.steps if wid != 5 else max(3, min(args.steps, 5))
    warm = _warm(torch, step, args.warmup if wid != 5 else 1, SETTLE_MS)
    # breakdown pass (events between all calls), then the timed steps with events around the dominant call only
    _log(f"[bench] per-call breakdown over {steps} steps")
    breakdown = Timer(torch, calls)
    for _ in range(steps):
        step(breakdown)
    torch.cuda.synchronize()
    breakdown.collect()
    per_call = {n: round(breakdown.median_ms(n), 4) for n in calls}
    dominant = max((n for n in ("fwd", "bwd_dq", "bwd_dkdv") if n in calls), key=lambda n: per_call[n])
    _log(f"[bench] timing {steps} steps")
    timer = Timer(torch, calls, only=(dominant,))
    t0 = time.perf_counter()
    for _ in range(steps):
        meta, _ = step(timer)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / steps * 1e3
    timer.collect()
    dominant_ms = round(timer.median_ms(dominant), 4)
    ms_eager = ms_per_step
    if args.graph:
        ms_per_step = time_graph(torch, step, steps)
    units, tiles = tile_work(meta, w.Tq, w.Tk, blk, torch)
    per_unit = 14.0 if w.train else 4.0
    step_flops = per_unit * units * w.d
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    attn_ms = sum(v for n, v in per_call.items() if n in ("block_meta", "fwd", "bwd_dq", "bwd_dkdv"))

    # dense causal at the original shape, same library
    _log("[bench] dense causal reference")
    dq_, dk_, dv_, do_ = dense_in
    nd = 1 if wid == 5 else max(3, steps // 4)

    def dense(b, t):
        if t:
            t.begin()
        o, lse = scfa.attn_fwd_lists(dq_, dk_, dv_, None, None, None, None, None, block=b, scale=sc)
        if t:
            t.mark()
        if w.train:
            g, delta = scfa.attn_bwd_dq_lists(dq_, dk_, dv_, o, lse, do_, None, None, None, None, None, block=b,
                                              scale=sc)
            scfa.attn_bwd_dkdv_lists(dq_, dk_, dv_, lse, do_, delta, None, None, None, None, None, block=b,
                                     scale=sc)
            if t:
                t.mark()

    dcalls = ["dense_fwd"] + (["dense_bwd"] if w.train else [])
    # at a million tokens one dense call takes seconds: only the workload's own block is timed there
    dense_ms, dense_blk, dense_by_block, dtimer = time_dense(torch, dense, DENSE_BLOCKS if wid != 5 else (blk,),
                                                             nd, 1, dcalls)
    nblk = (w.T + blk - 1) // blk

    # at d = 128 and block 128 the Hash-sparse forward runs each 128-query block as two 64-query groups
    fwd_tmpl = f"{w.d},64,true,128" if (w.mode != "qk" and w.d == 128 and blk == 128) else f"{w.d},{blk},true"
    kern = {"fwd": (f"k_fwd_bf16_ks<{'kQK' if w.mode == 'qk' else 'kHash'},{fwd_tmpl}>", 4.0 * units * w.d)}
    if w.train:
        kern["bwd_dq"] = (f"k_bwd_dq_bf16<kQK,{w.d},{blk},true>", 2.0 * units * w.d)
        kern["bwd_dkdv"] = (f"k_bwd_dkdv_bf16<kQK,{w.d},{blk},true,false>", 8.0 * units * w.d)
    out = {
        "metric": "effective TFLOP/s (executed tiles, % bf16 MFMA peak) + speedup vs dense causal",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "breakdown_steps": steps,
        "ms_per_step": round(ms_per_step, 4),
        "step_launch": "one HIP graph replay per step" if args.graph else "eager",
        "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, seeded keep sets and Gaussian LSH rotations)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "kept": w.n_keep, "d": w.d, "block": blk,
                   "n_buckets": w.n_buckets, "train": w.train, "step_calls": calls, "tile_rule": "exact"},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "executed_tiles": tiles,
        "dense_causal_tiles": w.B * w.H * nblk * (nblk + 1) // 2,
        "attention_only_tflops": round(step_flops / (attn_ms * 1e-3) / 1e12, 3),
        "dense_causal_ms": round(dense_ms, 4),
        "dense_causal_block": dense_blk,
        "dense_causal_ms_by_block": dense_by_block,
        "speedup_vs_dense_causal": round(dense_ms / ms_per_step, 3),
        "speedup_vs_dense_causal_attention_only": round(dense_ms / attn_ms, 3),
        "per_call_ms": per_call,
        "step_median_ms_events": round(breakdown.step_median_ms(), 4),
        "per_call_stat": f"median of {steps} HIP-event samples per call, from {steps} eager steps run before the "
                         f"timed ones (the timed steps record events only around {dominant})",
        "dense_per_call_ms": {n: round(dtimer.median_ms(n), 4) for n in dcalls},
        "roofline": _roofline(kern[dominant][0], kern[dominant][1], dominant_ms),
        "kernel_rooflines": {n: _roofline(kn, fl, per_call[n]) for n, (kn, fl) in kern.items()},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps before the timed ones (about 40 are needed before clocks settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-causal reference (short profiled runs)")
    ap.add_argument("--copy-sorted", action="store_true",
                    help="copy Q, dO, K, V into sorted order in the sorts (default: attention reads them through "
                         "the sort permutations)")
    ap.add_argument("--stored-ds", action="store_true",
                    help="backward with stored dS: the dK/dV kernel keeps each tile's dS and dQ is computed from it "
                         "(default: the dQ kernel recomputes S, P and dP, which measures faster on this workload)")
    ap.add_argument("--range-lists", action="store_true",
                    help="build the tile lists with the bucket-range rule only (keep tiles that hold no valid pair)")
    ap.add_argument("--workload", type=int, default=WORKLOAD_ID,
                    help="2, 3 or 5: that workload's line instead of the default (4) benchmark line")
    ap.add_argument("--sweep-nb", type=str, default="", metavar="LIST",
                    help="comma-separated bucket counts: one JSON line per count instead of the benchmark line")
    ap.add_argument("--sweep-drop", type=str, default="", metavar="LIST", help="comma-separated drop rates")
    ap.add_argument("--sweep-T", type=str, default="", metavar="LIST", help="comma-separated sequence lengths")
    ap.add_argument("--sweep-ragged", action="store_true",
                    help="QK-sparse heads with their own kept counts: packed heads against the padded layout")
    ap.add_argument("--measure-rows", action="store_true",
                    help="time the row gather / scatter calls instead of the step (one JSON line)")
    ap.add_argument("--graph", action="store_true",
                    help="--workload lines: time the step as one HIP graph replay (per-call times stay eager)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB (fp32) before the warmup, for counter scaling")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path has no multi-GPU code); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch

    import sparse_causal_attention_amd as scfa
    from gen import WORKLOADS

    if args.sweep_drop:
        sweep_drop(scfa, torch, [float(x) for x in args.sweep_drop.split(",")], args)
        return
    if args.sweep_ragged:
        sweep_ragged(scfa, torch, args)
        return
    if args.sweep_T:
        sweep_length(scfa, torch, [int(x) for x in args.sweep_T.split(",")], args)
        return
    if args.workload != WORKLOAD_ID:
        bench_workload(scfa, torch, args.workload, args)
        return

    w = WORKLOADS[WORKLOAD_ID]
    _log(f"[bench] workload {w.name}: generating inputs")
    q, k, v, do, R, qk = make_inputs(w, torch)
    torch.cuda.synchronize()
    if args.sweep_nb:
        sweep_buckets(scfa, torch, w, q, k, v, do, qk, [int(x) for x in args.sweep_nb.split(",")], args)
        return
    if args.measure_rows:
        measure_rows(scfa, torch, w, q, k, v, do, R, args)
        return

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        _log(f"[bench] calibration copy: {args.copy_calibration} MiB read + {args.copy_calibration} MiB written")
        del src, dst

    ds = prepare_ds(scfa, torch, w, q, k, R, qk, not args.range_lists, args.copy_sorted) if args.stored_ds else None
    _log("[bench] warmup")
    for _ in range(args.warmup):
        run_step(scfa, w, q, k, v, do, R, exact=not args.range_lists, copy_sorted=args.copy_sorted, qk=qk, ds=ds)
    torch.cuda.synchronize()

    # Per-call breakdown first: HIP events between all calls, on the stream the kernels run on, over
    # `steps` steps; it also picks the dominant attention kernel.  The timed steps then record events only
    # around that kernel (events between every call would add about 4 % to the step).
    calls = step_calls(args.copy_sorted, ds is not None)
    _log(f"[bench] per-call breakdown over {args.steps} steps")
    breakdown = Timer(torch, calls)
    for _ in range(args.steps):
        run_step(scfa, w, q, k, v, do, R, breakdown, exact=not args.range_lists, copy_sorted=args.copy_sorted,
                 qk=qk, ds=ds)
    torch.cuda.synchronize()
    breakdown.collect()
    per_call = {n: round(breakdown.median_ms(n), 4) for n in calls}
    dominant = max(("fwd", "bwd_dq", "bwd_dkdv"), key=lambda n: per_call[n])
    _log(f"[bench] timing {args.steps} steps")
    timer = Timer(torch, calls, only=(dominant,))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        meta, _ = run_step(scfa, w, q, k, v, do, R, timer, exact=not args.range_lists, copy_sorted=args.copy_sorted,
                           qk=qk, ds=ds)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    timer.collect()
    dominant_ms = round(timer.median_ms(dominant), 4)  # measured inside the timed region

    units, tiles = tile_work(meta, w.Tq, w.Tk, w.block, torch)
    step_flops = 14.0 * units * w.d
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    # tiles the bucket-range rule alone would visit (context; not timed)
    qh, qi, _, _, _ = scfa.lsh_bucket_sort(q, R, w.n_buckets)
    kh, ki, _, _, _ = scfa.lsh_bucket_sort(k, R, w.n_buckets)
    _, range_tiles = tile_work(scfa.block_meta(qi, ki, qh, kh, block=w.block, with_cols=False), w.Tq, w.Tk,
                               w.block, torch)

    dtimer = None
    dense_ms, dense_blk, dense_by_block = float("nan"), None, None
    if not args.no_dense:
        _log("[bench] dense causal reference")
        dense_ms, dense_blk, dense_by_block, dtimer = time_dense(
            torch, lambda b, t: run_dense(scfa, dataclasses.replace(w, block=b), q, k, v, do, t), DENSE_BLOCKS,
            max(3, args.steps // 4), max(1, min(args.warmup, 3)), DENSE_CALLS)

    attn_ms = sum(t for n, t in per_call.items() if not n.startswith("lsh"))
    rows_flag = "false" if args.copy_sorted else "true"
    if ds is None:
        # executed matrix flops per launch (tile units x d); the recomputing dQ kernel executes 6*d per tile unit,
        # of which 2*d (dS K) is algorithmic: it recomputes Q K^T and dO V^T, which the dK/dV kernel's 8*d counts
        kernel_flops = {"fwd": 4.0 * units * w.d, "bwd_dq": 6.0 * units * w.d, "bwd_dkdv": 8.0 * units * w.d}
        names = {"fwd": f"k_fwd_bf16_ks<kHash,64,64,{rows_flag}>", "bwd_dq": f"k_bwd_dq_bf16<kHash,64,64,{rows_flag}>",
                 "bwd_dkdv": f"k_bwd_dkdv_bf16<kHash,64,64,{rows_flag},false>"}
    else:
        # stored dS: dK/dV executes its 8*d per tile unit (all algorithmic) and writes each tile's dS;
        # dQ is dS K only (2*d per tile unit)
        kernel_flops = {"fwd": 4.0 * units * w.d, "bwd_dq": 2.0 * units * w.d, "bwd_dkdv": 8.0 * units * w.d}
        names = {"fwd": f"k_fwd_bf16_ks<kHash,64,64,{rows_flag}>", "bwd_dq": f"k_bwd_dq_ds_bf16<64,64,{rows_flag}>",
                 "bwd_dkdv": f"k_bwd_dkdv_bf16<kHash,64,64,{rows_flag},true>"}
    # algorithmic flops per launch: the dQ kernel's share is dS K only (2*d per tile unit)
    alg = {"fwd": 4.0 * units * w.d, "bwd_dq": 2.0 * units * w.d, "bwd_dkdv": 8.0 * units * w.d}
    achieved = alg[dominant] / (dominant_ms * 1e-3) / 1e12
    roofline = {
        "kernel": names[dominant],
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": (measured_traffic("range" if args.range_lists else "exact", "copied" if args.copy_sorted else
                                     "permuted", "stored_ds" if ds is not None else "recompute")
                    if dominant == "bwd_dkdv" else None),
        "avg_launch_ms": dominant_ms,
        "avg_launch_stat": f"median of {args.steps} HIP-event samples around its launch in the timed steps",
        "algorithmic_flops_per_launch": alg[dominant],
    }

    # each attention kernel's executed matrix flops per launch over its event time (context; "roofline" is
    # the dominant kernel's)
    kernel_rooflines = {
        n: {"kernel": names[n], "executed_tflops": round(kernel_flops[n] / (per_call[n] * 1e-3) / 1e12, 2),
            "executed_frac": round(kernel_flops[n] / (per_call[n] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": per_call[n], "executed_flops_per_launch": kernel_flops[n],
            "algorithmic_flops_per_launch": alg[n]}
        for n in kernel_flops}
    if ds is not None:
        # HBM-bound pieces of the stored-dS backward: the preprocess reads O and dO and writes D and lse*log2 e;
        # the dQ kernel reads each tile's dS once (2 bytes per tile unit)
        prep_bytes = w.B * w.H * w.Tq * (2 * 2 * w.d + 4 + 4 + 8)
        dq_bytes = 2.0 * units
        kernel_rooflines["bwd_prep"] = {"kernel": "k_bwd_prep<64>", "bound": "hbm", "avg_launch_ms": per_call["bwd_prep"],
                                        "algorithmic_bytes_per_launch": prep_bytes,
                                        "GBps": round(prep_bytes / (per_call["bwd_prep"] * 1e-3) / 1e9, 1),
                                        "frac_hbm": round(prep_bytes / (per_call["bwd_prep"] * 1e-3) / 1e9 /
                                                          PEAK_HBM_GBS, 4)}
        kernel_rooflines["bwd_dq"].update({"ds_bytes_per_launch": dq_bytes,
                                           "ds_GBps": round(dq_bytes / (per_call["bwd_dq"] * 1e-3) / 1e9, 1)})

    cpu = None
    if not args.no_cpu_baseline:
        _log("[bench] cpu oracle baseline (fp64, heads until the sample is long enough)")
        cpu = cpu_baseline(w, units / (w.B * w.H))

    out = {
        "metric": "effective TFLOP/s (executed tiles, % bf16 MFMA peak) + speedup vs dense causal",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "breakdown_steps": args.steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, seeded Gaussian LSH rotations)",
        "config": {
            "workload": w.name,
            "B": w.B,
            "H": w.H,
            "T": w.T,
            "d": w.d,
            "block": w.block,
            "n_buckets": w.n_buckets,
            "step": ("lsh+sort(Q,dO) + lsh+sort(K,V) + block lists + fwd + bwd" if args.copy_sorted else
                     "lsh+sort of Q and K (one call over the stacked [2B,H,T,d] tensor) + block lists + fwd + bwd, "
                     "rows read through the sort permutations, outputs written at the caller's rows"),
            "tile_rule": "range" if args.range_lists else "exact",
            "rows": "copied" if args.copy_sorted else "permuted",
            "outputs": meta["outputs"],
            "backward": "stored dS (dQ from the dK/dV kernel's dS tiles)" if ds is not None else
                        "recompute (dQ kernel recomputes S, P, dP)",
        },
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "executed_tiles": tiles,
        "range_rule_tiles": range_tiles,
        "dense_causal_tiles": w.B * w.H * (w.T // w.block) * (w.T // w.block + 1) // 2,
        "attention_only_tflops": round(step_flops / (attn_ms * 1e-3) / 1e12, 3),
        "dense_causal_ms": None if args.no_dense else round(dense_ms, 4),
        "dense_causal_block": dense_blk,
        "dense_causal_ms_by_block": dense_by_block,
        "speedup_vs_dense_causal": None if args.no_dense else round(dense_ms / ms_per_step, 3),
        "speedup_vs_dense_causal_excl_lsh": None if args.no_dense else round(dense_ms / attn_ms, 3),
        "per_call_ms": per_call,
        "step_median_ms_events": round(breakdown.step_median_ms(), 4),
        "per_call_stat": f"median of {args.steps} HIP-event samples per call, from {args.steps} steps run just "
                         f"before the timed ones (these record events between all calls; the timed steps only "
                         f"around {dominant})",
        "dense_per_call_ms": None if args.no_dense else {n: round(dtimer.median_ms(n), 4) for n in DENSE_CALLS},
        "roofline": roofline,
        "kernel_rooflines": kernel_rooflines,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
