#!/usr/bin/env python3
"""Bench: draft-head decode attention over a very long paged KV cache, one MI355X.

One step = one draft_attn_decode call: the device-side work decomposition, the
split-K streaming pass over every visible K/V block and the log-sum-exp merge
(a second kernel, or the tail of the streaming kernel on the single-launch
path, which the library picks for small steps). Inputs (seeded, synthetic,
bf16) are resident in HBM before timing starts. Each timed step is one eager
call through a prepared binding (arguments marshalled once, one C call per
step). --graph instead times replays of the call captured in a HIP graph; on
this software stack a replay costs more than an eager call.

Default workload: the million-token draft step (1 sequence, 2^20 cached keys in
16-token blocks behind a shuffled block table, 32 query / 8 kv heads, d = 128,
8 draft tokens, 1% high-norm needle keys), full attention over the whole
cache -- the read that grows with context. Printed: one JSON line with
  value       KV GB/s of the whole step (algorithmic K+V bytes / wall time)
  roofline    the streaming pass alone: algorithmic bytes / its mean duration
              (HIP events recorded by the library around that launch, in a
              second loop of the same calls so the timed steps carry none), against
              the 8 TB/s HBM peak; traffic = FETCH_SIZE + WRITE_SIZE bytes per
              launch from rocprofv3 counters (profiles/traffic.json), when they
              were taken on the current kernel source
  step_us_hot / step_us_cold  median, p10 and p90 of whole-call durations
              (torch events on the call's stream), the cold ones with the 256 MB
              Infinity Cache flushed by a 512 MiB write before each call
  copy_ceiling  a plain 1 GiB device copy's read + write rate in the same run
  cpu_baseline  the fp64 NumPy oracle on a bounded sample of the same step,
              timed on this host's cores (BLAS threads pinned to them)
Options select other workloads and modes for sweeps; --gpus above 1 is refused.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["draft_attention_amd/csrc/decode.hip", "draft_attention_amd/csrc/plan.h",
                  "draft_attention_amd/csrc/lanes.h", "draft_attention_amd/csrc/draft_part.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="needles_1m")
    ap.add_argument("--run", type=int, default=0, help="index into the workload's mode list")
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--launch", default="auto", choices=["auto", "two_pass", "single"])
    ap.add_argument("--window", type=int, default=None, help="override the run's window (window / fold modes)")
    ap.add_argument("--contiguous-blocks", action="store_true",
                    help="allocate each sequence's blocks in order instead of the shuffled block table")
    ap.add_argument("--op", default="decode", choices=["decode", "append", "merge_draft", "decode_draft"],
                    help="decode (the hot path, default) or one of the NEXT-row kernels")
    ap.add_argument("--case", default=None, help="append: decode | prefill; merge_draft: 1m | batch16; decode_draft: window_128k | window_1m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the call captured in a HIP graph instead of eager calls")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def kernel_source_hash(read=None) -> str:
    """sha256 of the streaming kernel's sources with // comments and blank lines
    removed, so that a comment edit does not retire the recorded counters."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel), "rb") as f:
                text = f.read().decode()
        else:
            text = read(rel)
        for line in text.splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def visible_keys(L, mode, window=0, n_sink=0, **_):
    """Keys whose K and V a step must read (the visible set's size)."""
    if mode == "window":
        return min(L, n_sink + window)
    return L


class HipEvents:
    """hipEvent_t handles from the HIP runtime that torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def calib_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 3}), flush=True)


def make_workload_inputs(w, seed, fold, shuffle=True):
    import torch

    import synth
    return synth.make_inputs(ctx_lens=w.ctx_lens, T=w.T, Hq=w.Hq, Hkv=w.Hkv, d=w.d, seed=seed,
                             device=torch.device("cuda:0"), fold=fold, needle_frac=w.needle_frac, fill="zero",
                             shuffle=shuffle)


def time_workload(w, kw, steps, warmup, seed, split, want_events=True, graph=False, launch="auto", shuffle=True,
                  want_dist=None, x=None, floor=False, min_warm_s=0.0):
    """Time `steps` decode calls on inputs generated on the GPU (or given as x); returns
    a result dict. want_events: the streaming pass's mean duration from the library's
    HIP events, in a second loop of the same calls; want_dist: whole-call hot and cold
    duration distributions (default: as want_events); floor: also time the call's
    launch shape with empty kernels, one and two of them, in the same eager loop."""
    import torch

    import draft_attention_amd as da

    if want_dist is None:
        want_dist = want_events
    dev = torch.device("cuda:0")
    if x is None:
        x = make_workload_inputs(w, seed, kw["mode"] == "fold", shuffle)
    side = x["k_side"] if kw["mode"] == "fold" else None
    out = torch.empty((len(w.ctx_lens), w.T, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((len(w.ctx_lens), w.T, w.Hq), dtype=torch.float32, device=dev)
    p = da.make_params(num_seqs=len(w.ctx_lens), num_draft_tokens=w.T, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                       head_dim=w.d, num_blocks=x["k_cache"].shape[0],
                       max_blocks_per_seq=x["block_table"].shape[1], split_keys=split, rope_theta=w.rope_theta,
                       launch=launch, **kw)
    ws = torch.empty(da.workspace_size(p, w.ctx_lens), dtype=torch.uint8, device=dev)
    _, chunk = da.plan(p, w.ctx_lens)
    launch_used = da.launch_of(p, w.ctx_lens)
    ev = HipEvents() if want_events else None
    pairs = [(ev.create(), ev.create()) for _ in range(steps)] if ev else [None] * steps

    call = da.prepare(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], k_side=side,
                      ctx_lens=w.ctx_lens, out=out, lse=lse, workspace=ws, rope_theta=w.rope_theta,
                      split_keys=split, launch=launch, **kw)

    def step(pe):
        call(prof_events=pe)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    if min_warm_s > 0:
        # further untimed steps until min_warm_s of them have run (the
        # secondary workloads: steady clocks, whatever ran before them)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            for _ in range(4):
                step(None)
            torch.cuda.synchronize()
    # Timed eager steps.
    t0 = time.perf_counter()
    for k in range(steps):
        step(None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_eager = (t1 - t0) * 1e3 / steps
    pass1 = None
    if ev:
        # The same calls again, the streaming kernel bracketed by HIP events.
        for k in range(steps):
            step(pairs[k])
        torch.cuda.synchronize()
        durs = [ev.elapsed_ms(a, b) for a, b in pairs]
        pass1 = sum(durs) / len(durs)
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
    floors = None
    if floor:
        # The same eager loop over the call's launch shape with empty kernels
        # that take the real kernels' argument blocks.
        floors = {}
        for nk in (1, 2):
            fcall = da.prepare_launch_floor(p, w.ctx_lens, nk)
            for _ in range(warmup):
                fcall()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fcall()
            torch.cuda.synchronize()
            floors[nk] = (time.perf_counter() - t0) * 1e3 / steps
    # Whole-call durations from torch events on the call's stream: the
    # distribution of hot steps, then cold steps with the 256 MB Infinity Cache
    # flushed by a 512 MiB write before each call.
    dist = cold = None
    if want_dist:
        import statistics

        def pct(v, q):
            v = sorted(v)
            return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record()
            step(None)
            b.record()
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) * 1e3 for a, b in evs]
        dist = dict(median=round(statistics.median(d), 2), p10=round(pct(d, 0.1), 2), p90=round(pct(d, 0.9), 2))
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        d = []
        for k in range(min(steps, 20)):
            flush.fill_(k & 0xFF)
            a, b = evs[k]
            a.record()
            step(None)
            b.record()
            torch.cuda.synchronize()
            d.append(a.elapsed_time(b) * 1e3)
        cold = dict(median=round(statistics.median(d), 2), p10=round(pct(d, 0.1), 2), p90=round(pct(d, 0.9), 2))
        del flush
    ms = ms_eager
    ms_graph = None
    if graph:
        # One step captured in a HIP graph and replayed: the whole call's GPU work
        # without the host's per-call launch cost, as a serving loop runs it.
        # The prepared call enqueues on the stream it was prepared with; under
        # capture it must go to the capturing stream, so it is named at each call.
        side_stream = torch.cuda.Stream()
        side_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side_stream):
            call(stream=side_stream.cuda_stream)
        torch.cuda.current_stream().wait_stream(side_stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(stream=torch.cuda.current_stream().cuda_stream)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_graph = ms = (t1 - t0) * 1e3 / steps
        del g
    keys = sum(visible_keys(L, **kw) for L in w.ctx_lens) * w.Hkv
    bytes_ = keys * 4 * w.d
    res = dict(x=x, kw=kw, ms=ms, ms_eager=ms_eager, pass1_ms=pass1, bytes=bytes_, keys=keys // w.Hkv, chunk=chunk,
               launch=launch_used, dist=dist, cold=cold, floors=floors,
               torch_ok=bool(torch.isfinite(out).all().item()))
    return res


def rate_entry(r):
    """Secondary-line entry of one timed workload: whole-step rate and, when timed,
    the streaming pass's duration and rate against the 8 TB/s peak."""
    gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    e = dict(ms_per_step=round(r["ms"], 5), draft_steps_per_s=round(1e3 / r["ms"], 1), kv_gbs=round(gbs, 1),
             pct_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 2), launch=r["launch"], split_keys=r["chunk"])
    if r["pass1_ms"]:
        p1 = r["bytes"] / (r["pass1_ms"] * 1e-3) / 1e9
        e.update(pass1_us=round(r["pass1_ms"] * 1e3, 2), pass1_gbs=round(p1, 1),
                 pass1_frac=round(p1 / HBM_PEAK_GBS, 4))
    if r["floors"]:
        f1, f2 = r["floors"][1] * 1e3, r["floors"][2] * 1e3
        step = r["ms"] * 1e3
        floor = f2 if r["launch"] == "two_pass" else f1
        e.update(floor_one_kernel_us=round(f1, 2), floor_two_kernels_us=round(f2, 2),
                 above_floor_us=round(step - floor, 2),
                 floor_note="the call's launch shape (grids, LDS, argument block sizes) with empty kernels, "
                            "same eager loop; above_floor is the step minus the floor of its own kernel count")
    return e


def copy_ceiling():
    """Read + write rate of a plain 1 GiB device copy (torch copy_), timed with events."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    del src, dst
    return dict(kernel="torch copy_ of 1 GiB", read_plus_write_gbs=round(2 * n / (ms * 1e-3) / 1e9, 1))


def cpu_baseline(w, kw, x, budget_s):
    """fp64 oracle on whole kv heads of the same step until the budget is spent, with the
    BLAS threads pinned to this process's cores."""
    import contextlib

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        limit, threads = contextlib.nullcontext(), 1
    G = w.Hq // w.Hkv
    table = x["block_table"].cpu().numpy()
    with limit:
        done_bytes, spent, heads = _oracle_heads(w, kw, x, budget_s, G, table)
    step_s = spent * w.Hkv / heads
    return dict(value=done_bytes / spent / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                s_per_step=round(step_s, 3),
                keys_per_s=round(sum(visible_keys(L, **kw) for L in w.ctx_lens) / step_s, 1),
                sample=f"{heads} of {w.Hkv} kv heads of the same step (all {sum(w.ctx_lens)} keys each), "
                       f"fp64 NumPy on {cores} host cores, {spent:.1f} s")


def _oracle_heads(w, kw, x, budget_s, G, table):
    import oracle

    done_bytes, spent, heads = 0, 0.0, 0
    for g in range(w.Hkv):
        q = x["q"][:, :, g * G:(g + 1) * G].float().cpu().numpy()
        k = x["k_cache"][:, g:g + 1].float().cpu().numpy()
        v = x["v_cache"][:, g:g + 1].float().cpu().numpy()
        ks = None if x["k_side"] is None else x["k_side"][:, g:g + 1].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.decode(q, k, v, table, w.ctx_lens, k_side=ks, rope_theta=w.rope_theta, **kw)
        spent += time.perf_counter() - t0
        heads += 1
        done_bytes += sum(visible_keys(L, **kw) for L in w.ctx_lens) * 4 * w.d
        del q, k, v, ks
        if spent >= budget_s:
            break
    return done_bytes, spent, heads


def traffic_for(tag):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(tag)
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _event_mean_us(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e6 / steps
    return a.elapsed_time(b) * 1e3 / steps, wall


def append_inputs(case, seed):
    """Inputs of the KV append (draft_attn_append) with the FOLD side cache. Cases: 'decode'
    writes the accepted tokens of a draft step (16 sequences x 8 tokens at ragged positions);
    'prefill' writes a 64K-token chunk of one sequence. Algorithmic bytes per token and kv
    head: read k_new and v_new, write the rotated key, the side key and the value, 10 * d
    bytes."""
    import torch

    import synth

    Hkv, d = 8, 128
    if case == "decode":
        pos = synth.ragged_lengths(16, 32768, 524288, seed)
        n_new = 8
    else:
        pos, n_new = [1000], 65536
    B = len(pos)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    spans = [list(range(p // 16, (p + n_new - 1) // 16 + 1)) for p in pos]
    MB = max(sp[-1] for sp in spans) + 1
    table = torch.full((B, MB), -1, dtype=torch.int32)
    nb = 0
    for b, sp in enumerate(spans):
        table[b, sp] = torch.arange(nb, nb + len(sp), dtype=torch.int32)
        nb += len(sp)
    table = table.to(dev)
    kc = torch.zeros((nb, Hkv, d // 8, 16, 8), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((nb, Hkv, d, 16), dtype=torch.bfloat16, device=dev)
    ks = torch.zeros_like(kc)
    kn = torch.randn((B, n_new, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, n_new, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    posd = torch.tensor(pos, dtype=torch.int32, device=dev)
    return dict(pos=pos, n_new=n_new, B=B, Hkv=Hkv, d=d, table=table, kc=kc, vc=vc, ks=ks, kn=kn, vn=vn, posd=posd,
                nbytes=B * n_new * Hkv * 10 * d)


def time_append(case, steps, warmup, seed):
    """Inputs, mean and wall µs per append call (HIP events around each call), GB/s."""
    import draft_attention_amd as da

    x = append_inputs(case, seed)
    call = da.prepare_append(x["kn"], x["vn"], x["table"], x["posd"], x["kc"], x["vc"], x["ks"], rope="neox",
                             rope_theta=5e5, pos_host=x["pos"])
    us, wall = _event_mean_us(call, steps, warmup)
    return x, us, wall, x["nbytes"] / (us * 1e-6) / 1e9


def bench_append(args):
    """KV append (draft_attn_append) with the FOLD side cache; cases as in append_inputs."""
    case = args.case or "prefill"
    x, us, wall, gbs = time_append(case, args.steps, args.warmup, args.seed)
    pos, n_new, B, Hkv, d = x["pos"], x["n_new"], x["B"], x["Hkv"], x["d"]
    table, kc, vc, ks, kn, vn = x["table"], x["kc"], x["vc"], x["ks"], x["kn"], x["vn"]
    nbytes = x["nbytes"]
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nb_s = min(B, 2) if case == "decode" else 1
        ns = n_new if case == "decode" else 4096
        kn_s, vn_s = kn[:nb_s, :ns].double().cpu().numpy(), vn[:nb_s, :ns].double().cpu().numpy()
        top = max(int(table[b, (pos[b] + ns - 1) // 16]) for b in range(nb_s)) + 1   # blocks the sample touches
        pools = [t[:top].double().cpu().numpy() for t in (kc, vc, ks)]
        t0 = time.perf_counter()
        oracle.append(kn_s, vn_s, table[:nb_s].cpu().numpy(), pos[:nb_s], *pools, rope="neox", rope_theta=5e5)
        spent = time.perf_counter() - t0
        cpu = dict(value=round(nb_s * ns * Hkv * 10 * d / spent / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                   sample=f"{nb_s} sequence(s) x {ns} tokens x {Hkv} kv heads, fp64 NumPy, {spent:.2f} s")
    line = {"metric": "KV append GB/s (rotated key + side key + value writes)", "value": round(gbs, 2),
            "unit": "GB/s", "op": "append", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "us_per_call": round(us, 2), "us_per_call_wall": round(wall, 2), "higher_is_better": True,
            "dtype": "bf16", "data": "synthetic",
            "config": {"case": case, "num_seqs": B, "num_new": n_new, "kv_heads": Hkv, "head_dim": d,
                       "side_cache": True, "positions": pos if B <= 4 else f"{B} ragged"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "append_kernel",
                         "bytes_per_launch": nbytes},
            "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def bench_merge_draft(args):
    """Draft-token self-attention merged into a decode result (draft_attn_merge_draft).
    Cases: '1m' (1 sequence, 8 draft tokens, 32/8 heads) and 'batch16' (16 sequences, 4
    draft tokens). Algorithmic bytes: q, the draft keys and values, out and lse read and
    written once."""
    import torch

    import draft_attention_amd as da

    case = args.case or "1m"
    B, T = (1, 8) if case == "1m" else (16, 4)
    Hq, Hkv, d = 32, 8, 128
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(args.seed)
    q = torch.randn((B, T, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    kd = torch.randn((B, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vd = torch.randn((B, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.randn((B, T, Hq, d), generator=g, device=dev)
    lse = torch.randn((B, T, Hq), generator=g, device=dev)
    lens = [1 << 20] * B if case == "1m" else [100000 + 1000 * b for b in range(B)]
    ctx = torch.tensor(lens, dtype=torch.int32, device=dev)

    call = da.prepare_merge_draft(q, kd, vd, ctx, out, lse, num_blocks=1 << 17, max_blocks_per_seq=1 << 16,
                                  num_kv_heads=Hkv, ctx_lens=lens)

    us, wall = _event_mean_us(call, args.steps, args.warmup)
    nbytes = B * T * (Hq * d * 2 + 2 * Hkv * d * 2 + 2 * Hq * d * 4 + 2 * Hq * 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    line = {"metric": "draft self-attention merge: us per call", "value": round(us, 2), "unit": "us",
            "op": "merge_draft", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "us_per_call_wall": round(wall, 2), "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"case": case, "num_seqs": B, "draft_tokens": T, "q_heads": Hq, "kv_heads": Hkv,
                       "head_dim": d},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None, "kernel": "merge_draft_kernel",
                         "bytes_per_launch": nbytes, "note": "a few hundred KB per call: launch- and latency-bound"},
            "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def bench_decode_draft(args):
    """A draft step's whole attention: the cache part (draft_attn_decode) merged with
    the draft tokens' causal part, as two calls (decode, then merge_draft: three
    kernels) against the fused call (draft_attn_decode_draft: two kernels). Cases:
    'window_128k' (WINDOW 2048 + 4 sinks at 131072 keys, 4 draft tokens) and
    'window_1m' (WINDOW 4096 + 4 at 2^20 keys, 8 draft tokens); 32/8 heads, d = 128.
    Reports us per step for both, eager calls."""
    import torch

    import draft_attention_amd as da
    import synth

    case = args.case or "window_128k"
    res = time_decode_draft(case, args.steps, args.warmup, args.seed)
    t1, t2, w1, w2 = res["fused_us"], res["two_calls_us"], res["fused_wall_us"], res["two_calls_wall_us"]
    L, T, W, Hq, Hkv, d = res["L"], res["T"], res["W"], 32, 8, 128
    line = {"metric": "draft step attention with draft tokens: us per step", "value": round(t1, 2), "unit": "us",
            "op": "decode_draft", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "us_per_step_fused": round(t1, 2), "us_per_step_two_calls": round(t2, 2),
            "us_per_step_wall_fused": round(w1, 2), "us_per_step_wall_two_calls": round(w2, 2),
            "config": {"case": case, "ctx_len": L, "draft_tokens": T, "window": W, "n_sink": 4, "q_heads": Hq,
                       "kv_heads": Hkv, "head_dim": d},
            "roofline": None, "cpu_baseline": None,
            "note": "latency-bound steps: the fused call saves the separate merge launch"}
    print(json.dumps(line), flush=True)


def time_decode_draft(case, steps, warmup, seed):
    """Window step with the step's draft tokens, as two calls (decode, then merge_draft)
    and as the fused call; event-timed means and wall times per step, in us."""
    import torch

    import draft_attention_amd as da
    import synth

    L, T, W = (131072, 4, 2048) if case == "window_128k" else (1 << 20, 8, 4096)
    Hq, Hkv, d = 32, 8, 128
    dev = torch.device("cuda:0")
    x = synth.make_inputs(ctx_lens=[L], T=T, Hq=Hq, Hkv=Hkv, d=d, seed=seed, device=dev, fill="zero")
    g = torch.Generator(device=dev).manual_seed(seed)
    kd = torch.randn((1, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vd = torch.randn((1, T, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    kw = dict(mode="window", window=W, n_sink=4, ctx_lens=[L])
    dec = da.prepare(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], **kw)
    mrg = da.prepare_merge_draft(x["q"], kd, vd, x["ctx_len"], dec.out, dec.lse, num_blocks=x["k_cache"].shape[0],
                                 max_blocks_per_seq=x["block_table"].shape[1], num_kv_heads=Hkv, mode="window",
                                 window=W, n_sink=4, ctx_lens=[L])
    fused = da.prepare(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_len"], k_draft=kd, v_draft=vd,
                       **kw)

    def two_calls():
        dec()
        mrg()

    t2, w2 = _event_mean_us(two_calls, steps, warmup)
    t1, w1 = _event_mean_us(fused, steps, warmup)
    del x
    return dict(fused_us=t1, two_calls_us=t2, fused_wall_us=w1, two_calls_wall_us=w2, L=L, T=T, W=W)


def secondary_rates(wl, args):
    """The metric's other draft-step rates, each with its streaming pass's duration
    and fraction of 8 TB/s: FULL at 128K; the windowed steps (window + sinks) at
    128K and 1M against their launch floor; FOLD at 256K for every alpha/beta pair
    of that workload; the 16-sequence ragged batch with query scaling, FULL and
    FOLD; the window steps with the step's draft tokens (fused and as two
    calls); and the KV append of a draft step's accepted tokens and of a 64K-token
    prefill chunk. Inputs are generated once per workload; each decode entry
    warms up with the run's W steps and then for at least 200 ms more before it
    is timed."""
    import torch

    out = {}
    steps, warmup, seed = args.steps, args.warmup, args.seed

    def run(name, kws, label):
        w = wl[name]
        x = make_workload_inputs(w, seed, any(k["mode"] == "fold" for k in kws))
        for kw in kws:
            r = time_workload(w, kw, steps, warmup, seed, 0, want_events=True, want_dist=False, graph=args.graph,
                              x=x, floor=kw["mode"] == "window", min_warm_s=0.2)
            out[label(w, kw)] = rate_entry(r)
            del r
        del x
        torch.cuda.empty_cache()

    mode_label = lambda w, kw: f"{w.name}/{kw['mode']}"  # noqa: E731
    run("llama8b_128k", wl["llama8b_128k"].runs, mode_label)
    run("needles_1m", [wl["needles_1m"].runs[1]], mode_label)
    run("fold_256k", wl["fold_256k"].runs,
        lambda w, kw: f"{w.name}/fold alpha={kw['alpha']:g} beta={kw['beta']:g}")
    run("batch16_ragged", wl["batch16_ragged"].runs,
        lambda w, kw: f"{w.name}/{kw['mode']} kappa={kw['kappa']:g}")
    for case in ("window_128k", "window_1m"):
        d = time_decode_draft(case, steps, warmup, seed)
        out[f"decode_draft/{case}"] = dict(fused_us=round(d["fused_us"], 2),
                                           two_calls_us=round(d["two_calls_us"], 2),
                                           draft_tokens=d["T"], window=d["W"], ctx_len=d["L"])
    for case in ("decode", "prefill"):
        x, us, _, gbs = time_append(case, steps, warmup, seed)
        out[f"append/{case}"] = dict(us_per_call=round(us, 2), gbs=round(gbs, 1),
                                     pct_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 2), num_seqs=x["B"],
                                     num_new=x["n_new"], bytes=x["nbytes"])
        del x
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported. The path shards by sequence, "
              "kv head or key range, but no multi-GPU path is implemented.",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.op == "append":
        bench_append(args)
        return
    if args.op == "merge_draft":
        bench_merge_draft(args)
        return
    if args.op == "decode_draft":
        bench_decode_draft(args)
        return
    import synth

    wl = synth.workloads(args.seed)
    w = wl[args.workload]
    kw = dict(w.runs[args.run])
    if args.window is not None:
        kw["window"] = args.window
    r = time_workload(w, kw, args.steps, args.warmup, args.seed, args.split_keys, graph=args.graph,
                      launch=args.launch, shuffle=not args.contiguous_blocks, floor=kw["mode"] == "window")
    gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    p1 = r["bytes"] / (r["pass1_ms"] * 1e-3) / 1e9
    tag = f"{w.name}/{kw['mode']}"
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, kw, r["x"], args.cpu_budget_s)
        cpu["value"] = round(cpu["value"], 4)
    torch_ok = r["torch_ok"]
    # The headline's inputs are released before the other workloads are
    # generated and timed (with them still held, the 128K window step measured
    # 12.9 us here against 10.7 us on its own).
    del r["x"]
    import torch
    torch.cuda.empty_cache()
    secondary = {}
    if not args.no_secondary and w.name == "needles_1m":
        secondary = secondary_rates(wl, args)
    mode_str = kw["mode"] + ("" if kw["mode"] == "full" else f" W={kw.get('window', 0)} sinks={kw.get('n_sink', 0)}")
    line = {
        "metric": "draft-attention KV GB/s & % HBM peak; draft steps/s at 128K and 1M context",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "ms_per_step_eager": round(r["ms_eager"], 5),
        "timing": "replays of one call captured in a HIP graph" if args.graph else "eager calls",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": mode_str, "num_seqs": len(w.ctx_lens),
                   "ctx_len": w.ctx_lens[0] if len(w.ctx_lens) == 1 else w.ctx_lens,
                   "draft_tokens": w.T, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "block_size": 16,
                   "split_keys": r["chunk"], "launch": r["launch"],
                   "block_table": "in order" if args.contiguous_blocks else "shuffled",
                   "alpha": kw.get("alpha", 1.0), "beta": kw.get("beta", 0.0),
                   "kappa": kw.get("kappa", 0.0)},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "draft_steps_per_s": round(1e3 / r["ms"], 2),
        "keys_per_s": round(r["keys"] / (r["ms"] * 1e-3), 1),
        "kv_bytes_per_step": r["bytes"],
        "roofline": {"bound": "hbm", "achieved": round(p1, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(p1 / HBM_PEAK_GBS, 4), "traffic": traffic_for(tag),
                     "kernel": ("pass1_kernel (split-K K/V streaming)" if r["launch"] == "two_pass" else
                                "pass1_kernel (split-K K/V streaming + in-kernel merge, single launch)"),
                     "mean_launch_ms": round(r["pass1_ms"], 5)},
        "step_us_hot": r["dist"],
        "step_us_cold": r["cold"],
        "copy_ceiling": copy_ceiling() if not args.no_secondary else None,
        "secondary": secondary,
        "floor": (None if not r["floors"] else rate_entry(r)),
        "cpu_baseline": cpu,
    }
    if not torch_ok:
        line["error"] = "non-finite output"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
