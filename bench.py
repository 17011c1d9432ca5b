#!/usr/bin/env python3
"""Benchmark: one decode step (append + grouped-query attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa_8b]

A step is the whole hot path over one batch: kvc_decode_step, i.e. the append
(rotate and store the new key, store the value, rotate q) and the attention of
every query head over its group's cache (the streaming kernel, which also does
the append, and, when a sequence has several splits, the merge kernel).  Inputs are resident in HBM before timing starts.
To keep the 256 MB Infinity Cache from serving the cache between steps, R
replicas of the KV cache (R * bytes >= 2 GB) are used in turn.

Prints one JSON line: `value` is the algorithmic KV bytes one step must read
(sum_b L_b * H_kv * d * 2 * 2 bytes) divided by the measured step time.
`roofline` rates the streaming kernel alone (per-launch time from HIP events the
library attaches to that kernel's launch on its stream) against 8 TB/s.
`cpu_baseline` is the CPU oracle timed on the host on the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MALL_DEFEAT_BYTES = 2 << 30
# committed rocprofv3 counter runs per (cache kind, workload), and the sources
# the streaming kernel is built from: counters taken on other versions of them
# do not describe the current kernel
_CSRC = os.path.join(ROOT, "mqa_decode_attention_amd", "csrc")
_COMMON = ("kvc_mfma_common.h", "kvc_device.h", "kvc_internal.h")
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries of the streaming kernel per
# configuration (profiles/), and the sources of that kernel they were taken on
TRAFFIC = {
    ("native", "gqa_8b"): ("decode_gqa_8b_traffic.json", ("kvc_decode_mfma.hip",) + _COMMON),
    ("u8", "gqa_8b"): ("decode_u8_gqa_8b_traffic.json", ("kvc_decode_u8.hip",) + _COMMON),
    ("native", "mqa_ragged"): ("decode_mqa_ragged_traffic.json", ("kvc_decode_mfma.hip", "kvc_decode.hip") + _COMMON),
    ("native", "long_gqa"): ("decode_long_gqa_traffic.json", ("kvc_decode_mfma.hip",) + _COMMON),
    ("native", "paged_gqa"): ("decode_paged_gqa_traffic.json", ("kvc_decode_mfma.hip", "kvc_decode.hip") + _COMMON),
    ("u8", "paged_gqa"): ("decode_u8_paged_gqa_traffic.json", ("kvc_decode_u8.hip",) + _COMMON),
    ("native", "tiny_mha"): ("decode_tiny_mha_traffic.json", ("kvc_decode.hip",) + _COMMON),
    ("native", "spec_gqa"): ("decode_spec_gqa_traffic.json",
                             ("kvc_decode_mfma.hip", "kvc_append.hip", "kvc_decode.hip") + _COMMON),
    ("native", "mla_latent"): ("decode_mla_latent_traffic.json", ("kvc_mla.hip",) + _COMMON),
    ("fp8_e4m3", "gqa_8b"): ("decode_fp8_e4m3_gqa_8b_traffic.json", ("kvc_decode_u8.hip",) + _COMMON),
}


def kv_read_bytes(seq_lens, H_kv, d, elem_bytes):
    """Bytes of K and V a decode step must read: sum_b L_b * H_kv * d * 2 * e."""
    return int(sum(int(L) for L in seq_lens)) * H_kv * d * 2 * elem_bytes


def attended(seq_lens, window):
    """Tokens each sequence attends: all of them, or the last `window`."""
    return [min(int(L), window) if window > 0 else int(L) for L in seq_lens]


def kvc_q8_dtype(kind):
    """The torch dtype naming an 8-bit cache kind in the library's plan queries."""
    import torch
    return {"u8": torch.uint8, "fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2}[kind]


def kv_read_bytes_u8(seq_lens, H_kv, d):
    """The same for the quantized cache: d codes plus an 8-byte (step, zero
    point) pair per token, KV head and tensor."""
    return int(sum(int(L) for L in seq_lens)) * H_kv * (d + 8) * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gqa_8b",
                    help="gqa_8b (default), mqa_ragged, long_gqa, paged_gqa, tiny_mha, spec_gqa, or the latent "
                         "cache mla_latent")
    ap.add_argument("--split-tokens", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window of W tokens (kvc_decode_step_window over the full cache; 0 = none)")
    ap.add_argument("--ring", action="store_true",
                    help="with --window: the cache is a ring of W slots holding each sequence's window")
    ap.add_argument("--kv-cache", choices=("native", "u8", "fp8_e4m3", "fp8_e5m2"), default="native",
                    help="native: the workload's dtype (kvc_decode_step); u8: the uint8 cache (kvc_decode_step_u8 "
                         "on codes drawn by workloads.draw_quantized); fp8_e4m3 / fp8_e5m2: the FP8 cache "
                         "(kvc_decode_step_fp8 on codes drawn by workloads.draw_fp8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only measure the streaming-read ceiling (kvc_hbm_read_probe)")
    return ap.parse_args()


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_for_current_kernel(kind: str, workload: str):
    """HBM bytes per launch of the streaming kernel from the committed rocprofv3
    counter runs of this workload, if they were taken on the current kernel
    sources; else None."""
    if (kind, workload) not in TRAFFIC:
        return None
    name, sources = TRAFFIC[(kind, workload)]
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            t = json.load(f)
        if t.get("kernel_sources_sha256") == kernel_source_hash(sources):
            return t.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def calibrate_copy(nbytes: int) -> None:
    """A plain device copy of known size (read nbytes, write nbytes), five times:
    what FETCH_SIZE / WRITE_SIZE report for it scales the counters of the kernel."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "copies": 5}))


def cpu_threads() -> int:
    """Host cores for the all-cores oracle figure: the CPUs this process may
    run on, at most OMP_NUM_THREADS (the share of the host one GPU gets)."""
    n = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(n, cap) if cap > 0 else n)


# The task the forked oracle workers run (set before the pool forks, so each
# worker inherits it with the step's inputs; nothing large is sent to them).
_CPU_TASK = None


def _cpu_task(i):
    _CPU_TASK(i)
    return 0


def _cpu_noop(_):
    return 0


def time_cpu_tasks(task, n_tasks: int, procs: int) -> float:
    """Seconds to run task(0), ..., task(n_tasks - 1): in this process when
    procs == 1, else spread over `procs` forked worker processes (started
    before the clock runs).  One BLAS thread per process either way.  Must run
    before this process touches the GPU: a forked copy of a process holding a
    GPU context must not exist."""
    global _CPU_TASK
    from threadpoolctl import threadpool_limits

    _CPU_TASK = task
    with threadpool_limits(limits=1):
        if procs <= 1:
            t0 = time.perf_counter()
            for i in range(n_tasks):
                task(i)
            return time.perf_counter() - t0
        import multiprocessing as mp
        with mp.get_context("fork").Pool(procs) as pool:
            pool.map(_cpu_noop, range(4 * procs))
            t0 = time.perf_counter()
            pool.map(_cpu_task, range(n_tasks), chunksize=1)
            return time.perf_counter() - t0


def _np_store(t, dt):
    import numpy as np
    import torch
    t = t.contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()


def oracle_tasks(x, kind: str, window: int = 0, qc=None):
    """The step's CPU oracle as independent (sequence, KV head) tasks: each
    appends the group's new token(s) and attends its G query heads, on its own
    slices of the inputs (a paged cache: the sequence's rows gathered through
    its block table first).  Returns (task, n_tasks, kv_bytes, what)."""
    import numpy as np

    import oracle as O

    w = x.workload
    dt, G, H_kv = w.dtype, w.G, w.H_kv
    e = 2 if dt == "bf16" else 4
    cos, sin = x.rope_cos.numpy(), x.rope_sin.numpy()
    cached = x.cached.numpy()
    n_new = w.new_tokens
    q, kn, vn = _np_store(x.q, dt), _np_store(x.k_new, dt), _np_store(x.v_new, dt)
    tbl = x.block_table.numpy() if w.paged else None
    if kind != "native":
        import oracle.kvc_fp8_oracle as FO
        import oracle.kvc_quant_oracle as QO
        arrs = [a.numpy() for a in (qc.k_codes, qc.k_sz, qc.v_codes, qc.v_sz)]
    else:
        kc, vc = _np_store(x.k_cache, dt), _np_store(x.v_cache, dt)

    def rows(a, b, j, L):
        """[1, 1, L, ...] rows of group (b, j): a slice, or a gather from a pool."""
        if w.paged:
            return O.gather_paged(a, tbl, w.block_size, b, L)[None, j:j + 1]
        return a[b:b + 1, j:j + 1, :L]

    def task(i):
        b, j = divmod(i, H_kv)
        hs = slice(j * G, (j + 1) * G)
        c = cached[b:b + 1]
        L = int(cached[b]) + n_new
        if kind == "u8":
            g = [rows(a, b, j, L) for a in arrs]
            g = QO.append_contiguous_u8(*g, c, kn[b:b + 1, j:j + 1], vn[b:b + 1, j:j + 1], cos, sin, dt,
                                        q=q[b:b + 1, hs])
            QO.decode_attention_u8(g[4], *g[:4], [L], dt)
        elif kind != "native":
            fmt = kind[4:]
            g = [rows(a, b, j, L) for a in arrs]
            g = FO.append_contiguous_fp8(*g, c, kn[b:b + 1, j:j + 1], vn[b:b + 1, j:j + 1], cos, sin, dt, fmt,
                                         q=q[b:b + 1, hs])
            FO.decode_attention_fp8(g[4], *g[:4], [L], dt, fmt)
        elif n_new > 1:
            import oracle.kvc_multi_oracle as MO
            k2, v2, q2 = MO.append_multi(rows(kc, b, j, L), rows(vc, b, j, L), c, kn[b:b + 1, :, j:j + 1],
                                         vn[b:b + 1, :, j:j + 1], cos, sin, dt, q=q[b:b + 1, :, hs])
            MO.decode_attention_multi(q2, k2, v2, [L], dt, window)
        else:
            k2, v2, q2 = O.append_contiguous(rows(kc, b, j, L), rows(vc, b, j, L), c, kn[b:b + 1, j:j + 1],
                                             vn[b:b + 1, j:j + 1], cos, sin, dt, q=q[b:b + 1, hs])
            if window:
                import oracle.kvc_window_oracle as WO
                WO.decode_attention_window(q2, k2, v2, [L], window, dt)
            else:
                O.decode_attention(q2, k2, v2, [L], dt)

    lens = (cached + n_new).tolist()
    if kind != "native":
        nbytes = kv_read_bytes_u8(lens, H_kv, w.d)
        what = ("uint8" if kind == "u8" else kind.upper().replace("_", " ")) + " cache, append + attention"
    else:
        span = window + n_new - 1 if window else 0
        nbytes = kv_read_bytes(attended(lens, span), H_kv, w.d, e)
        what = (f"append of {n_new} tokens + their attention" if n_new > 1 else "append + attention") + \
            (f" over the last {window} tokens" if window else "") + (", rows gathered through the block table"
                                                                     if w.paged else "")
    return task, w.B * H_kv, nbytes, what


def oracle_tasks_mla(x):
    """The latent-cache oracle as one task per sequence (the listing's per-head
    up-projection of that sequence's latents, then the attention)."""
    import oracle.kvc_mla_oracle as MO

    w = x.workload
    cache = _np_store(x.cache, "bf16")
    n = {k: _np_store(getattr(x, k), "bf16") for k in ("w_uk", "b_uk", "w_uv", "b_uv")}
    q, ckv, kr = _np_store(x.q, "bf16"), _np_store(x.c_kv_new, "bf16"), _np_store(x.k_rope_new, "bf16")
    cached = x.cached.numpy()

    def task(b):
        c2 = MO.append_mla(cache[b:b + 1], cached[b:b + 1], ckv[b:b + 1], kr[b:b + 1])
        MO.decode_attention_mla(q[b:b + 1], c2, cached[b:b + 1] + 1, n["w_uk"], n["b_uk"], n["w_uv"], n["b_uv"],
                                w.d_latent, w.dtype)

    nbytes = latent_read_bytes(cached + 1, w.d_latent, 2)
    return task, w.B, nbytes, "append + per-head up-projection of the latents + attention"


def cpu_baselines(tasks, name: str, B: int) -> dict:
    """The oracle (as it stands, float64 numpy) timed on the host on the whole
    step: over all cores this process may use (one worker process per core,
    tasks handed out one at a time), and on one core."""
    task, n, nbytes, what = tasks
    procs = cpu_threads()
    out = {}
    for key, p in (("cpu_baseline", procs), ("cpu_baseline_one_core", 1)):
        sec = time_cpu_tasks(task, n, p)
        how = "one process" if p == 1 else f"{p} worker processes, one per core"
        out[key] = {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": p, "kind": "oracle",
                    "sample": f"all {B} sequences of {name} as {n} independent tasks ({what}; float64, numpy, "
                              f"one BLAS thread each; {how}), {sec:.2f} s"}
    return out


def latent_read_bytes(seq_lens, d_latent, elem_bytes):
    """Bytes of the latent cache a step must read: sum_b L_b * d_latent * e (the
    rope part of each row is stored but not attended)."""
    return int(sum(int(L) for L in seq_lens)) * d_latent * elem_bytes


def bench_mla(args, W) -> dict:
    """One decode step over a latent cache: kvc_decode_step_mla (append + absorbed
    queries, the streaming pass, the split merge, the value up-projection)."""
    import torch

    import mqa_decode_attention_amd as kvc

    w = W.MLA_WORKLOADS[args.workload]
    x = W.draw_mla(w)
    # the host oracle first: its worker processes are forked before this
    # process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baselines(oracle_tasks_mla(x), w.name, w.B)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvc.load()
    probe = read_probe(reps=5)      # also brings the part to its working clocks before the timed steps
    e = 2
    kv_bytes = latent_read_bytes(x.seq_lens.tolist(), w.d_latent, e)
    weight_bytes = 2 * w.H * w.d_k * w.d_latent * e
    cache_bytes = x.cache.numel() * e
    R = max(1, min(64, -(-MALL_DEFEAT_BYTES // cache_bytes)))
    caches = [x.cache.to(dev) for _ in range(R)]
    q, ckv, kr = x.q.to(dev), x.c_kv_new.to(dev), x.k_rope_new.to(dev)
    wk, wv, bv = x.w_uk.to(dev), x.w_uv.to(dev), x.b_uv.to(dev)
    pos = x.cached.to(dev)
    max_len = int(x.seq_lens.max())
    out = torch.empty((w.B, w.H, w.d_k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        if ev is not None:
            kvc.profile_next_decode(ev[0], ev[1])
        kvc.decode_step_mla(q, caches[i % R], pos, ckv, kr, max_len, wk, wv, bv, out=out,
                            split_tokens=args.split_tokens)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_ms, batch_stats, wall = timed_steps(step, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    timing = "start and stop events attached to each launch"
    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    check_kernel_timing(achieved, w.name)
    value = kv_bytes / (step_ms * 1e-3) / 1e9
    res = {
        "metric": "GQA decode-attn KV read GB/s (% of MI355X HBM peak); us per decode step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) latents and queries, NaN past each sequence's length; up-projections "
                "drawn as nn.Linear initialises them)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "d_k": w.d_k, "d_latent": w.d_latent,
                   "rope_dim": w.rope_dim, "cached_tokens": [w.cached_lo, w.cached_hi], "layout": "contiguous",
                   "kv_bytes_per_step": kv_bytes, "weight_bytes_per_step": weight_bytes, "cache_replicas": R,
                   "split_tokens": kvc.mla_split_tokens(w.B, w.H, w.d_latent, max_len, args.split_tokens),
                   "split_choice": "explicit" if args.split_tokens else "library"},
        "us_per_step": round(step_ms * 1e3, 2),
        "step_ms_batches": batch_stats,
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_median": round(sorted(dec_ms)[len(dec_ms) // 2] * 1e3, 2),
        # the absorbed form's score and PV multiply-adds: 4 * d_latent per
        # (head, token)
        "decode_tflops": round(4 * w.H * w.d_latent * int(x.seq_lens.sum()) / (dec_avg_ms * 1e-3) / 1e12, 2),
        "flops_per_step": 4 * w.H * w.d_latent * int(x.seq_lens.sum()),
        "hbm_pct_step": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for_current_kernel("native", w.name),
                     "kernel": "mla_decode_kernel (streaming pass over the latent rows; the absorbed queries with "
                               "the append, the split merge and the value up-projection are separate small kernels)",
                     "bytes_per_launch": kv_bytes, "launch_timing": timing},
        "wall_s_timed": round(wall, 4),
    }
    ceil_nt = probe["nontemporal"]["best_gbs"]
    res["read_ceiling"] = {"probe": "kvc_hbm_read_probe, 4 GiB, best grid",
                           "default_policy_gbs": probe["default"]["best_gbs"], "nontemporal_gbs": ceil_nt,
                           "kernel_frac_of_ceiling": round(achieved / ceil_nt, 4)}
    if cpu:
        res.update(cpu)
    return res


def timed_steps(step, steps: int, batches: int = 5):
    """Time `steps` back-to-back steps between two events on the current
    stream, with events at batch boundaries inside: (ms per step over all of
    them, {median, min, max} ms per step over the batches)."""
    import torch

    n = max(1, min(batches, steps))
    bounds = [round(k * steps / n) for k in range(n + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record()
    for k in range(n):
        for i in range(bounds[k], bounds[k + 1]):
            step(i)
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = sorted(evs[k].elapsed_time(evs[k + 1]) / max(1, bounds[k + 1] - bounds[k]) for k in range(n))
    total = evs[0].elapsed_time(evs[n]) / steps
    stats = {"batches": n, "median_ms": round(per[len(per) // 2], 5), "min_ms": round(per[0], 5),
             "max_ms": round(per[-1], 5)}
    return total, stats, wall


def check_kernel_timing(achieved_gbs: float, what: str) -> None:
    """The per-launch events must bracket the streaming kernel: a rate above the
    HBM peak means they did not (e.g. a step path that never asked the library
    for them) and the figure would be meaningless."""
    if achieved_gbs > 1.05 * HBM_PEAK_GBS:
        print(f"bench.py: {what}: {achieved_gbs:.0f} GB/s exceeds the HBM peak; the per-launch timing events "
              "did not bracket the streaming kernel", file=sys.stderr)
        sys.exit(3)


def read_probe(gib: int = 4, reps: int = 10) -> dict:
    """Streaming-read rate of kvc_hbm_read_probe over a 4 GiB buffer (far beyond
    the 256 MB Infinity Cache), best of several grid sizes, with the default and
    with the non-temporal cache policy (the one the decode kernels use)."""
    import ctypes

    import torch

    import mqa_decode_attention_amd as kvc

    lib = kvc.load()
    nbytes = gib << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    for nt in (0, 1):
        best = {}
        for wgs in (1024, 2048, 4096, 8192):
            sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
            args = (ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), wgs, nt, st)
            rc = lib.kvc_hbm_read_probe(*args)
            assert rc == 0, lib.kvc_last_error()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                lib.kvc_hbm_read_probe(*args)
            b.record()
            torch.cuda.synchronize()
            best[wgs] = round(nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
        res["nontemporal" if nt else "default"] = {"gbs": best, "best_gbs": max(best.values())}
    res["buffer_gib"] = gib
    return res


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.read_probe:
        print(json.dumps(read_probe()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence and KV head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W

    # (device_count does not create a GPU context: the host oracle's worker
    # processes are forked before anything does)
    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.workload in W.MLA_WORKLOADS:
        if args.window or args.ring or args.kv_cache != "native":
            print("the latent-cache workload has no window or quantized variant", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(bench_mla(args, W)), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    x = W.draw(w)
    u8 = args.kv_cache != "native"         # an 8-bit cache: uint8 or FP8 codes with per-vector pairs
    fmt = {"u8": None, "fp8_e4m3": "e4m3", "fp8_e5m2": "e5m2"}.get(args.kv_cache)
    win = args.window
    multi = w.new_tokens > 1          # several new tokens per sequence: append_multi + decode_attn_multi
    if multi and (u8 or args.ring):
        print("multi-token workloads run on the native full cache", file=sys.stderr)
        sys.exit(2)
    if (win or args.ring) and (u8 or w.paged and args.ring or args.ring and win <= 0):
        print("--window applies to the native cache; --ring needs --window and a contiguous workload",
              file=sys.stderr)
        sys.exit(2)
    e = 2 if w.dtype == "bf16" else 4
    qc = (W.draw_quantized(x) if fmt is None else W.draw_fp8(x, fmt)) if u8 else None
    # the host oracle first: its worker processes are forked before this
    # process touches the GPU
    cpu = None if args.no_cpu_baseline else \
        cpu_baselines(oracle_tasks(x, args.kv_cache, win, qc), w.name, w.B)

    import mqa_decode_attention_amd as kvc

    kvc.load()   # fails loudly if libkvc.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probe = read_probe(reps=5)      # also brings the part to its working clocks before the timed steps
    if u8:
        kv_bytes = kv_read_bytes_u8(x.seq_lens.tolist(), w.H_kv, w.d)
        cache_bytes = (qc.k_codes.numel() + qc.k_sz.numel() * 4) * 2
    else:
        kv_bytes = kv_read_bytes(attended(x.seq_lens.tolist(), win + w.new_tokens - 1 if win else 0), w.H_kv, w.d, e)
        cache_bytes = x.k_cache.numel() * e * 2
    R = max(1, min(64, -(-MALL_DEFEAT_BYTES // cache_bytes)))

    if u8:
        ks = [(qc.k_codes.to(dev), qc.k_sz.to(dev)) for _ in range(R)]
        vs = [(qc.v_codes.to(dev), qc.v_sz.to(dev)) for _ in range(R)]
    elif args.ring:
        # a ring of W slots holding the window each sequence has before the
        # step (token t in slot t % W; slots never written stay NaN)
        rk = torch.full((w.B, w.H_kv, win, w.d), float("nan"), dtype=x.k_cache.dtype)
        rv = rk.clone()
        for b, c in enumerate(x.cached.tolist()):
            for t in range(max(0, c - win + 1), c):
                rk[b, :, t % win] = x.k_cache[b, :, t]
                rv[b, :, t % win] = x.v_cache[b, :, t]
        R = max(1, min(64, -(-MALL_DEFEAT_BYTES // (rk.numel() * e * 2))))
        ks = [rk.to(dev) for _ in range(R)]
        vs = [rv.to(dev) for _ in range(R)]
    else:
        ks = [x.k_cache.to(dev) for _ in range(R)]
        vs = [x.v_cache.to(dev) for _ in range(R)]
    q = x.q.to(dev)
    kn, vn = x.k_new.to(dev), x.v_new.to(dev)
    pos, lens = x.cached.to(dev), x.seq_lens.to(dev)
    cos, sin = x.rope_cos.to(dev), x.rope_sin.to(dev)
    tbl = x.block_table.to(dev) if w.paged else None
    max_len = int(x.seq_lens.max())
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    q_rot = torch.empty_like(q)
    q_work = q.clone()    # multi-token step: the append rotates the query in place (rotation keeps its norm)
    # the plain step (contiguous or paged cache): each replica's call checked
    # once, as a serving loop that reuses its buffers would; launching it is
    # then one foreign call
    prepared = None
    if u8:
        prepared = [kvc.prepare_decode_step_u8(q, ks[r][0], ks[r][1], vs[r][0], vs[r][1], pos, kn, vn, cos, sin,
                                               max_len, block_table=tbl, q_rot_out=q_rot, out=out,
                                               split_tokens=args.split_tokens, fmt=fmt)
                    for r in range(R)]
    elif not (multi or win):
        prepared = [kvc.prepare_decode_step(q, ks[r], vs[r], pos, kn, vn, cos, sin, max_len, block_table=tbl,
                                            q_rot_out=q_rot, out=out, split_tokens=args.split_tokens)
                    for r in range(R)]

    def step(i, ev=None):
        r = i % R
        if u8:
            if ev is not None:
                kvc.profile_next_decode(ev[0], ev[1])
            prepared[r]()
            return
        if multi:
            kvc.append_multi(ks[r], vs[r], pos, kn, vn, cos, sin, q=q_work, block_table=tbl)
            if ev is not None:
                kvc.profile_next_decode(ev[0], ev[1])
            kvc.decode_attn_multi(q_work, ks[r], vs[r], lens, max_len, win, block_table=tbl, out=out,
                                  split_tokens=args.split_tokens)
            return
        if ev is not None:
            kvc.profile_next_decode(ev[0], ev[1])
        if win:
            kvc.decode_step_window(q, ks[r], vs[r], pos, kn, vn, cos, sin, max_len, win, ring=args.ring,
                                   block_table=tbl, q_rot_out=q_rot, out=out, split_tokens=args.split_tokens)
            return
        prepared[r]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole-step timing: K steps back to back between two events (batch
    # boundaries marked inside), nothing else in between
    step_ms, batch_stats, wall = timed_steps(step, args.steps)

    # Per-launch duration of the streaming decode kernel: start and stop
    # events the library attaches to that kernel's launch on its stream
    # (hipExtLaunchKernel).  (In a plain run these agree with rocprofv3's
    # kernel durations within a few per cent; the attached events can
    # lengthen the launches they time - the quantized kernel's by about 10 % -
    # so the figure is an upper bound on the kernel's own time.)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:        # create the underlying HIP events
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    timing = "start and stop events attached to each launch"
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    dec_med_ms = sorted(dec_ms)[len(dec_ms) // 2]

    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    check_kernel_timing(achieved, w.name)
    value = kv_bytes / (step_ms * 1e-3) / 1e9
    traffic = None if (win or args.ring) else traffic_for_current_kernel(args.kv_cache, w.name)
    # algorithmic flops: score and PV multiply-adds, 4 * d per (query head,
    # attended token), for every new token's query
    att = attended(x.seq_lens.tolist(), win + w.new_tokens - 1 if win else 0)
    flops = 4 * w.d * w.H_q * w.new_tokens * int(sum(att))
    pool_tokens = x.k_cache.shape[0] * w.block_size if w.paged else 0

    res = {
        "metric": "GQA decode-attn KV read GB/s (% of MI355X HBM peak); us per decode step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded uint8 codes and per-vector (step, zero point) pairs of N(0,1)-like "
                 "vectors, NaN pairs past each sequence's length)") if args.kv_cache == "u8" else
                (f"synthetic (seeded FP8 {fmt.upper()} codes and per-vector (scale, 0) pairs of N(0,1)-like "
                 "vectors, NaN pairs past each sequence's length)") if u8 else
                "synthetic (seeded N(0,1), NaN past each sequence's length)",
        "config": {"workload": w.name + (f"_{args.kv_cache}" if u8 else "") + (f"_window{win}" if win else "") +
                               ("_ring" if args.ring else ""), "batch": w.B, "H_q": w.H_q, "H_kv": w.H_kv,
                   "head_dim": w.d, "cached_tokens": [w.cached_lo, w.cached_hi], "layout": w.layout,
                   "kv_cache": ("uint8 codes + float32 (step, zero point) per vector" if fmt is None else
                                f"FP8 {fmt.upper()} codes + float32 (scale, 0) per vector") if u8 else w.dtype,
                   "kv_bytes_per_step": kv_bytes, "cache_replicas": R,
                   "window": win, "ring": bool(args.ring), "new_tokens": w.new_tokens,
                   "split_tokens": (kvc.multi_split_tokens(x.q.dtype, w.B, w.new_tokens, w.H_q, w.H_kv, w.d, max_len,
                                                           win, args.split_tokens, pool_tokens=pool_tokens)
                                    if multi else
                                    kvc.split_tokens(kvc_q8_dtype(args.kv_cache) if u8 else x.q.dtype, w.B, w.H_q,
                                                     w.H_kv, w.d,
                                                     kvc.window_span(max_len, win, args.ring, win if args.ring else 0),
                                                     args.split_tokens, pool_tokens=pool_tokens)),
                   "split_choice": "explicit" if args.split_tokens else "library"},
        "us_per_step": round(step_ms * 1e3, 2),
        "step_ms_batches": batch_stats,
        "decode_us": round(dec_avg_ms * 1e3, 2),
        "decode_us_median": round(dec_med_ms * 1e3, 2),
        "decode_tflops": round(flops / (dec_avg_ms * 1e-3) / 1e12, 2),
        "flops_per_step": flops,
        "hbm_pct_step": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("decode_u8_kernel (streaming pass over the 8-bit codes with the fused append; a "
                                "one-round plan merges its splits in the same launch, else a small merge kernel "
                                "follows)") if u8 else
                               ("decode_mfma_kernel, multi-token rows (one pass over the cache for all new tokens' "
                                "queries; the append and the split merge are separate small kernels)") if multi else
                               ("decode_mfma_kernel (streaming pass with the fused append; a one-round plan merges "
                                "its splits in the same launch, else a small merge kernel follows)"),
                     "bytes_per_launch": kv_bytes, "launch_timing": timing},
        "wall_s_timed": round(wall, 4),
    }
    ceil_nt = probe["nontemporal"]["best_gbs"]
    res["read_ceiling"] = {"probe": "kvc_hbm_read_probe, 4 GiB, best grid",
                           "default_policy_gbs": probe["default"]["best_gbs"], "nontemporal_gbs": ceil_nt,
                           "kernel_frac_of_ceiling": round(achieved / ceil_nt, 4)}
    if cpu:
        res.update(cpu)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
