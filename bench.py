#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Prints ONE JSON line.  The headline workload is dense GQA decode over a
contiguous bf16 cache: B = 8 sequences, Hq = 32 query heads, Hkv = 8 kv-heads,
head dim 128, 32768 cached positions, split-KV chunks of 512.  A step is one
decode-attention call over the whole batch (every kernel of the call).

  value      = algorithmic bytes of a step / step time   (GB/s, KV read +
               query + output), inputs resident in HBM
  ms_per_step, us_per_step, pct_of_peak (of 8 TB/s)
  roofline   = the split-KV partial kernel alone (the dominant kernel), timed
               with HIP events on the launch stream: KV + query bytes per
               launch / mean launch time, against 8 TB/s
  cpu_baseline = the fp64 CPU oracle on a bounded sample of the same workload
  variants   = config 1, one sequence at 8K and 32K, dense at 128K, group
               sizes 1, 2, 8, 16 and 32 on the headline cache,
               the paged (one and four tokens), fixed-maximum, FFD, multi-row
               and cache-append entry points on their own workloads (same
               timing method)

K/V live in several copies that the timed steps rotate through, so each call
reads data that is not resident in the 256 MB last-level cache.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0       # MI355X HBM3E peak, GB/s
VARIANTS = ("config1", "dense_b1", "dense_128k", "groups", "paged", "paged_multi", "unified_max",
            "ffd", "ffd_peaked", "multi_row", "append")
METRIC = "us/decode step and achieved KV-read HBM GB/s (% of peak) at 32K-128K ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_partial_dense_b8_h32x8_d128_l32768.txt")
# everything that decides the partial kernel's code: its sources, the
# launch path and the compiler flags
KERNEL_SOURCES = ["long_context_decode_fd_amd/csrc/attn.hip",
                  "long_context_decode_fd_amd/csrc/splitkv.hpp",
                  "long_context_decode_fd_amd/csrc/common.hpp",
                  "long_context_decode_fd_amd/csrc/internal.hpp",
                  "long_context_decode_fd_amd/csrc/api.hip",
                  "long_context_decode_fd_amd/build.py"]
# (name, function) pairs filled by the timed legs: each function compares a
# sample of that leg's GPU output with the oracle (run in the CPU leg)
PARITY_SAMPLES = []


def parse_args():
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--copies", type=int, default=3, help="rotated K/V copies")
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="untimed run time before each extra workload's warm-up")
    p.add_argument("--no-variants", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device copy (counter scale for --pmc runs)")
    p.add_argument("--variants", default=",".join(VARIANTS),
                   help="comma-separated subset of the variant workloads to run")
    p.add_argument("--ffd-deltas", default=None,
                   help="comma-separated deltas for the FFD workloads (default 5,7)")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the partial kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def interleaved(timer, groups, steps, warmup, rounds=3):
    """Time several call groups in alternation, `rounds` times each, and keep
    the median per group (clock and power state drift over a run; measuring
    alternately keeps comparisons fair)."""
    res = {k: [] for k in groups}
    for _ in range(rounds):
        for k, calls in groups.items():
            res[k].append(timer.run(calls, steps, warmup))
    return {k: sorted(v, key=lambda t: t["ms"])[len(v) // 2] for k, v in res.items()}


class Timer:
    """Back-to-back calls on the current stream, timed with HIP events.

    `ms` is the mean over `steps` calls between one event before the first
    and one after the last (synchronized on both sides).  The spread (p10,
    p50, p90) comes from a second pass of back-to-back windows of 4 calls,
    an event between windows: the per-call mean of each window.  An event
    costs the stream about 3 us (FFD peaked workload: 64.4 us per call with
    an event after every call, 61.5 without), so events after every call
    would add their own cost and jitter to each step; per window of 4 the
    added cost is under 1 us per call.

    `settle_ms` (the extra workloads only; the headline step keeps exactly
    the warm-up it is given): before the warm-up calls, the calls run
    untimed for that much wall time.  The first ~100 back-to-back calls of a
    workload swing by up to 8 % on these GPUs (power-management and memory
    transients after idle periods or large allocations), which a warm-up of
    a few calls does not cover; a serving loop decodes in the settled
    state."""

    def __init__(self, torch, settle_ms=0.0):
        self.torch = torch
        self.settle_ms = settle_ms

    def run(self, calls, steps, warmup, settle=True):
        torch = self.torch
        n = len(calls)
        if settle and self.settle_ms > 0:
            t_end = time.perf_counter() + self.settle_ms * 1e-3
            i = 0
            while time.perf_counter() < t_end:
                for _ in range(8):
                    calls[i % n]()
                    i += 1
                torch.cuda.synchronize()
        for i in range(warmup):
            calls[i % n]()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(steps):
            calls[i % n]()
        e1.record(s)
        torch.cuda.synchronize()
        total = e0.elapsed_time(e1)
        win, nwin = 4, max(10, steps // 2)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
        ev[0].record(s)
        for w in range(nwin):
            for i in range(win):
                calls[(w * win + i) % n]()
            ev[w + 1].record(s)
        torch.cuda.synchronize()
        per = sorted(ev[w].elapsed_time(ev[w + 1]) / win for w in range(nwin))
        return dict(ms=total / steps, p10=per[len(per) // 10],
                    p50=per[len(per) // 2], p90=per[(9 * len(per)) // 10])


def vp(t):
    return C.c_void_p(t.data_ptr())


def check_rc(lib, rc):
    if rc != 0:
        raise RuntimeError(f"library call failed ({rc}): {lib.fd_last_error().decode()}")


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "dispatches": 3}), flush=True)


def dense_headline(torch, fd, W, args, timer):
    cfg = W.CONFIGS[2]
    B, Hq, Hkv, L, d, chunk = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["L"], cfg["d"], cfg["chunk"]
    case = W.config_case(2, device="cuda:0")
    ks = [case.k] + [case.k.clone() for _ in range(args.copies - 1)]
    vs = [case.v] + [case.v.clone() for _ in range(args.copies - 1)]
    lib = fd.lib()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    wsn = fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, chunk=chunk)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    scale = case.scale

    def mk_full(k, v):
        a = (fd.FD_BF16, vp(case.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, scale,
             chunk, vp(ws), C.byref(size), st)
        return lambda: lib.fd_decode_attn(*a)

    def mk_part(k, v):
        a = (fd.FD_BF16, vp(case.q), vp(k), vp(v), B, Hq, Hkv, L, d, scale, chunk, vp(ws),
             C.byref(size), st)
        return lambda: lib.fd_decode_attn_partials(*a)

    full = [mk_full(k, v) for k, v in zip(ks, vs)]
    part = [mk_part(k, v) for k, v in zip(ks, vs)]
    check_rc(lib, full[0]())
    check_rc(lib, part[0]())
    t_full = timer.run(full, args.steps, args.warmup, settle=False)
    t_part = timer.run(part, args.steps, args.warmup, settle=False)

    check_rc(lib, full[0]())
    sample_rows(torch, "config2 dense GQA bf16 (sequence 0, all 32 heads)", case.q[:1], case.k[:1],
                case.v[:1], out[:1], lse[:1], case.scale)

    kv_bytes = 2 * B * Hkv * L * d * 2
    q_bytes = B * Hq * d * 2
    out_bytes = B * Hq * d * 4 + B * Hq * 4
    step_bytes = kv_bytes + q_bytes + out_bytes
    part_bytes = kv_bytes + q_bytes
    achieved = gbs(part_bytes, t_part["ms"])
    return case, dict(
        t_full=t_full, t_part=t_part, step_bytes=step_bytes, part_bytes=part_bytes,
        value=gbs(step_bytes, t_full["ms"]), achieved=achieved,
        workload=dict(workload="dense GQA decode, contiguous bf16 KV cache", B=B, Hq=Hq,
                      Hkv=Hkv, head_dim=d, kv_len=L, chunk=chunk, n_chunks=L // chunk,
                      scale="1/sqrt(128)", kv_copies_rotated=args.copies))


def _host(t):
    """Exact host copy (bf16 stays bf16, fp32 stays fp32)."""
    return t.detach().to("cpu").clone()


def sample_rows(torch, name, q, k, v, out, lse, scale, tol=2e-3):
    """Register a dense-definition parity sample: q [b, Hq, d], k/v [b, Hkv,
    L, d] and the GPU's out/lse for those rows, copied to the host now."""
    q, k, v, o, l_ = _host(q), _host(k), _host(v), _host(out), _host(lse)

    def check():
        import numpy as np
        from oracle import flash_decoding as ofd
        f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
        ref, lref = ofd.dense_attention(f(q), f(k), f(v), scale)
        return _errs(np, f(o), f(l_), ref, lref, tol, q.shape[0] * q.shape[1])
    PARITY_SAMPLES.append((name, check))


def _errs(np, o, l_, ref, lref, tol, rows):
    eo = float(np.abs(o - ref).max())
    el = float(np.abs(l_ - lref).max())
    return dict(rows=int(rows), max_abs_err_out=eo, max_abs_err_lse=el, tol=tol,
                within_tol=bool(eo <= tol and el <= tol))


def variant_config1(torch, fd, W, args, timer):
    """Dense MHA fp32 (B 1, H 8, d 64, L 4096, chunk 1024: 4 chunks of 1024):
    16 MiB of K/V per copy, so it is timed twice: rotating 64 copies (1 GiB,
    every call reads from HBM) and on one copy (cache-resident after the
    first call).  A call this small is bound by launch latency."""
    c = W.config_case(1, device="cuda:0")
    B, Hq, d = c.q.shape
    Hkv, L = c.k.shape[1], c.k.shape[2]
    copies = 64
    ks = [c.k] + [c.k.clone() for _ in range(copies - 1)]
    vs = [c.v] + [c.v.clone() for _ in range(copies - 1)]
    lib = fd.lib()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    wsn = fd.workspace_bytes("fd_decode_attn", dt=fd.FD_F32, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d,
                             chunk=c.chunk)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for k, v in zip(ks, vs):
        a = (fd.FD_F32, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
             c.chunk, vp(ws), C.byref(size), st)
        calls.append(lambda a=a: lib.fd_decode_attn(*a))
    check_rc(lib, calls[0]())
    sample_rows(torch, "config1 dense MHA fp32 (all 8 heads)", c.q, c.k, c.v, out, lse, c.scale,
                tol=1e-5)
    t = interleaved(timer, {"cold": calls, "warm": calls[:1]}, args.steps, args.warmup)
    nbytes = 2 * B * Hkv * L * d * 4 + B * Hq * d * 4 + B * Hq * (d + 1) * 4
    res = dict(workload=f"dense MHA decode fp32, B={B}, H={Hq}, d={d}, L={L}, chunk={c.chunk}",
               bytes=nbytes)
    for key, note in (("cold", f"{copies} rotated K/V copies (1 GiB): HBM reads"),
                      ("warm", "one K/V copy: cache-resident after the first call")):
        res[key] = dict(us_per_step=round(t[key]["ms"] * 1e3, 2),
                        p10_us=round(t[key]["p10"] * 1e3, 2), p90_us=round(t[key]["p90"] * 1e3, 2),
                        gbs=round(gbs(nbytes, t[key]["ms"]), 1), note=note)
    return res


def cpu_baseline(torch, case, target_s):
    """fp64 oracle on whole sequences of the headline workload until about
    target_s seconds of oracle time; bf16 -> fp64 conversion excluded."""
    import numpy as np
    from oracle import flash_decoding as ofd
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, Hq, d = case.q.shape
    Hkv, L = case.k.shape[1], case.k.shape[2]
    G = Hq // Hkv
    # the whole headline step takes well under a second of oracle time, so the
    # step is repeated (whole passes over the B sequences, converted to fp64
    # once) until about target_s seconds of oracle time are spent
    t0 = time.perf_counter()
    seqs = [(case.q[b].to("cpu", torch.float64).numpy(),
             case.k[b].to("cpu", torch.float64).numpy(),
             case.v[b].to("cpu", torch.float64).numpy()) for b in range(B)]
    t_conv = time.perf_counter() - t0
    t_oracle, done, passes = 0.0, 0, 0
    while t_oracle < target_s:
        for qb, K, V in seqs:
            t1 = time.perf_counter()
            for h in range(Hq):
                ofd.attention_row(qb[h], K[h // G], V[h // G], case.scale)
            t_oracle += time.perf_counter() - t1
            done += 1
        passes += 1
    del seqs
    seq_bytes = 2 * Hkv * L * d * 2 + Hq * d * 2 + Hq * d * 4 + Hq * 4
    return dict(value=round(gbs(done * seq_bytes, t_oracle * 1e3), 4), unit="GB/s",
                cores=int(threads), kind="oracle",
                sample=(f"{passes} passes over the whole headline step ({B} sequences, all "
                        f"{Hq} query heads each); fp64 numpy oracle, {t_oracle:.2f} s; "
                        f"bf16->fp64 input conversion {t_conv:.2f} s excluded"),
                us_per_step_equiv=round(t_oracle / done * B * 1e6, 1),
                host_cpus=len(os.sched_getaffinity(0)))


def variant_dense_b1(torch, fd, W, args, timer):
    """One sequence at 8K and 32K positions (Hq 32, Hkv 8, d 128, chunk 512):
    fewer units than SIMDs, so the call splits its chunks further; 24 and 8
    rotated K/V copies (0.8 and 1.1 GB), so every call reads HBM."""
    res = dict(workload="dense GQA decode bf16, B=1, Hq=32, Hkv=8, d=128, chunk=512 "
                        "(short calls: splits shorter than the chunk)")
    for L, copies in ((8192, 24), (32768, 8)):
        B, Hq, Hkv, d, chunk = 1, 32, 8, 128, 512
        c = W.dense_case(B, Hq, Hkv, L, d, "bf16", chunk, seed=1201, device="cuda:0")
        ks = [c.k] + [c.k.clone() for _ in range(copies - 1)]
        vs = [c.v] + [c.v.clone() for _ in range(copies - 1)]
        lib = fd.lib()
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
        wsn = fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, chunk=chunk)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
        size = C.c_size_t(wsn)
        st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        calls = []
        for k, v in zip(ks, vs):
            a = (fd.FD_BF16, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d,
                 c.scale, chunk, vp(ws), C.byref(size), st)
            calls.append(lambda a=a: lib.fd_decode_attn(*a))
        check_rc(lib, calls[0]())
        t = timer.run(calls, args.steps, args.warmup)
        nbytes = 2 * B * Hkv * L * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
        res[f"L_{L}"] = dict(us_per_step=round(t["ms"] * 1e3, 2), p10_us=round(t["p10"] * 1e3, 2),
                             p90_us=round(t["p90"] * 1e3, 2), bytes=nbytes,
                             gbs=round(gbs(nbytes, t["ms"]), 1),
                             pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1))
        del ks, vs, c
    return res


def variant_dense_128k(torch, fd, W, args, timer):
    """Dense GQA decode at the long end of the 32K-128K range: B 2, L 131072
    (the same 1.07 GB of KV as the headline), chunk 512."""
    B, Hq, Hkv, L, d, chunk = 2, 32, 8, 131072, 128, 512
    c = W.dense_case(B, Hq, Hkv, L, d, "bf16", chunk, seed=1202, device="cuda:0")
    ks = [c.k] + [c.k.clone() for _ in range(args.copies - 1)]
    vs = [c.v] + [c.v.clone() for _ in range(args.copies - 1)]
    lib = fd.lib()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    wsn = fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, chunk=chunk)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for k, v in zip(ks, vs):
        a = (fd.FD_BF16, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
             chunk, vp(ws), C.byref(size), st)
        calls.append(lambda a=a: lib.fd_decode_attn(*a))
    check_rc(lib, calls[0]())
    t = timer.run(calls, args.steps, args.warmup)
    nbytes = 2 * B * Hkv * L * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
    return dict(workload=f"dense GQA decode bf16, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, L={L}, "
                         f"chunk={chunk}", us_per_step=round(t["ms"] * 1e3, 2),
                p10_us=round(t["p10"] * 1e3, 2), p90_us=round(t["p90"] * 1e3, 2), bytes=nbytes,
                gbs=round(gbs(nbytes, t["ms"]), 1),
                pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1))


def variant_groups(torch, fd, W, args, timer):
    """Single-query decode on the headline cache (B 8, Hkv 8, d 128, L 32768,
    chunk 512, bf16) with G = 1, 2, 8, 16 and 32 query heads per kv-head
    (Hq = 8 G): the vector kernel for G 1 and 2, the matrix-core kernel for
    G 8 (chosen: the vector kernel is issue-bound there), 16 and 32 (one and
    two query tiles)."""
    B, Hkv, L, d, chunk = 8, 8, 32768, 128, 512
    c = W.multi_case(B, 1, 32 * Hkv, Hkv, L, d, chunk=chunk, seed=1216, device="cuda:0")
    ks = [c.k] + [c.k.clone() for _ in range(args.copies - 1)]
    vs = [c.v] + [c.v.clone() for _ in range(args.copies - 1)]
    lib = fd.lib()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = dict(workload=f"dense decode bf16 by group size: B={B}, Hkv={Hkv}, d={d}, L={L}, "
                        f"chunk={chunk}, Hq = 8 G (G 1, 2: vector kernel; 8, 16, 32: "
                        f"matrix-core kernel)")
    for G in (1, 2, 8, 16, 32):
        Hq = G * Hkv
        q = c.q[:, 0, :Hq].contiguous()
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
        wsn = fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, chunk=chunk)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
        size = C.c_size_t(wsn)
        calls = []
        for k, v in zip(ks, vs):
            a = (fd.FD_BF16, vp(q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
                 chunk, vp(ws), C.byref(size), st)
            calls.append(lambda a=a: lib.fd_decode_attn(*a))
        check_rc(lib, calls[0]())
        t = timer.run(calls, args.steps, args.warmup)
        nbytes = 2 * B * Hkv * L * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
        res[f"G_{G}"] = dict(Hq=Hq, us_per_step=round(t["ms"] * 1e3, 2),
                             p10_us=round(t["p10"] * 1e3, 2), p90_us=round(t["p90"] * 1e3, 2),
                             bytes=nbytes, gbs=round(gbs(nbytes, t["ms"]), 1),
                             pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1))
    return res


def variant_multi(torch, fd, W, args, timer):
    """Multi-row decode on the headline shape (B 8, Hq 32, Hkv 8, d 128,
    L 32768, chunk 512) with M = 2, 4 and 8 new tokens per sequence (G*M = 8,
    16 and 32 query rows per kv-head, matrix-core kernel), beside M separate
    single-query calls on the same cache; each also at chunk 2048."""
    B, Hq, Hkv, L, d, chunk = 8, 32, 8, 32768, 128, 512
    base = W.multi_case(B, 8, Hq, Hkv, L, d, chunk=chunk, seed=102, device="cuda:0")
    ks = [base.k] + [base.k.clone() for _ in range(args.copies - 1)]
    vs = [base.v] + [base.v.clone() for _ in range(args.copies - 1)]
    lib = fd.lib()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    kv_bytes = 2 * B * Hkv * L * d * 2
    res = dict(workload=f"multi-row decode bf16, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, L={L}, "
                        f"chunk={chunk}, token r sees positions 0..L-M+r")
    t_single = None
    for M in (1, 2, 4, 8):
        q = base.q[:, :M].contiguous()
        out = torch.empty((B, M, Hq, d), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device="cuda:0")
        wsn = fd.workspace_bytes("fd_decode_attn_multi", B=B, M=M, Hq=Hq, Hkv=Hkv, L=L, d=d,
                                 chunk=chunk)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
        size = C.c_size_t(wsn)
        calls = []
        for k, v in zip(ks, vs):
            a = (fd.FD_BF16, vp(q), vp(k), vp(v), vp(out), vp(lse), B, M, Hq, Hkv, L, d,
                 base.scale, chunk, vp(ws), C.byref(size), st)
            calls.append(lambda a=a: lib.fd_decode_attn_multi(*a))
        check_rc(lib, calls[0]())
        t = timer.run(calls, args.steps, args.warmup)
        nbytes = kv_bytes + B * M * Hq * d * 2 + B * M * Hq * (d + 1) * 4
        if M == 1:
            t_single = t["ms"]
            continue
        res[f"M_{M}"] = dict(rows_per_kv_head=M * Hq // Hkv, us_per_step=round(t["ms"] * 1e3, 2),
                             p10_us=round(t["p10"] * 1e3, 2), p90_us=round(t["p90"] * 1e3, 2),
                             bytes=nbytes, gbs=round(gbs(nbytes, t["ms"]), 1),
                             pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1),
                             m_single_query_calls_us=round(M * t_single * 1e3, 2),
                             speedup_vs_single_calls=round(M * t_single / t["ms"], 2))
        # the same call with chunks of 2048 (16 per sequence): a quarter of the
        # partials (G*M rows of d+2 floats per chunk) to write and merge
        ch2 = 2048
        wsn2 = fd.workspace_bytes("fd_decode_attn_multi", B=B, M=M, Hq=Hq, Hkv=Hkv, L=L, d=d,
                                  chunk=ch2)
        ws2 = torch.empty(wsn2, dtype=torch.uint8, device="cuda:0")
        size2 = C.c_size_t(wsn2)
        calls2 = []
        for k, v in zip(ks, vs):
            a = (fd.FD_BF16, vp(q), vp(k), vp(v), vp(out), vp(lse), B, M, Hq, Hkv, L, d,
                 base.scale, ch2, vp(ws2), C.byref(size2), st)
            calls2.append(lambda a=a: lib.fd_decode_attn_multi(*a))
        check_rc(lib, calls2[0]())
        t2 = timer.run(calls2, args.steps, args.warmup)
        res[f"M_{M}"].update(us_per_step_chunk2048=round(t2["ms"] * 1e3, 2),
                             pct_of_peak_chunk2048=round(
                                 100 * gbs(nbytes, t2["ms"]) / PEAK_GBS, 1))
    return res


def variant_append(torch, fd, W, args, timer):
    """Cache append of the decode step's own token (M = 1) on the headline
    shapes: contiguous cache (B = 8, Hkv = 8, d = 128) and a paged pool with
    per-sequence positions (B = 16).  Latency-bound: 32-64 KiB per call."""
    import numpy as np
    dev = "cuda:0"
    bf = torch.bfloat16
    lib = fd.lib()
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    B, Hkv, d, L_cap, M = 8, 8, 128, 4096, 1
    kc = torch.zeros((B, Hkv, L_cap, d), dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    kn = torch.randn((B, Hkv, M, d), device=dev).to(bf)
    vn = torch.randn((B, Hkv, M, d), device=dev).to(bf)
    a = (fd.FD_BF16, vp(kn), vp(vn), vp(kc), vp(vc), B, Hkv, M, L_cap, d, L_cap - 1, st)
    call = lambda: lib.fd_kv_append(*a)  # noqa: E731
    check_rc(lib, call())
    t = timer.run([call], args.steps, args.warmup)
    PB, page, maxp, P = 16, 16, 1024, 16 * 1024
    kp = torch.zeros((P, Hkv, page, d), dtype=bf, device=dev)
    vpool = torch.zeros_like(kp)
    rs = np.random.default_rng(0)
    table = torch.as_tensor(rs.permutation(P).reshape(PB, maxp).astype(np.int32), device=dev)
    pos = torch.as_tensor(rs.integers(1024, maxp * page, size=PB).astype(np.int32), device=dev)
    kn2 = torch.randn((PB, Hkv, M, d), device=dev).to(bf)
    vn2 = torch.randn((PB, Hkv, M, d), device=dev).to(bf)
    a2 = (fd.FD_BF16, vp(kn2), vp(vn2), vp(kp), vp(vpool), vp(table), vp(pos), PB, Hkv, M, d,
          page, maxp, P, st)
    call2 = lambda: lib.fd_kv_append_paged(*a2)  # noqa: E731
    check_rc(lib, call2())
    t2 = timer.run([call2], args.steps, args.warmup)
    nb = lambda b: 2 * 2 * b * Hkv * M * d * 2  # noqa: E731  (read + write, K and V)
    return dict(workload="append of one new token's K/V rows, bf16, Hkv=8, d=128",
                contiguous=dict(B=B, us_per_call=round(t["ms"] * 1e3, 2), bytes=nb(B)),
                paged=dict(B=PB, page=page, us_per_call=round(t2["ms"] * 1e3, 2),
                           bytes=nb(PB)))


def variant_paged(torch, fd, W, args, timer):
    cfg = W.CONFIGS[3]
    c = W.config_case(3, device="cuda:0")
    B, Hq, d = c.q.shape
    Hkv = c.k_pool.shape[1]
    lens = c.meta["lens"]
    max_len = int(max(lens))
    lib = fd.lib()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    wsn = fd.workspace_bytes("fd_decode_attn_paged", B=B, Hq=Hq, Hkv=Hkv, d=d, page=c.page,
                             max_pages=c.block_table.shape[1], max_seq_len=max_len,
                             chunk=c.chunk)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = (fd.FD_BF16, vp(c.q), vp(c.k_pool), vp(c.v_pool), vp(c.block_table), vp(c.seq_lens),
         vp(out), vp(lse), B, Hq, Hkv, d, c.page, c.block_table.shape[1], c.k_pool.shape[0],
         max_len, c.scale, c.chunk, vp(ws), C.byref(size), st)
    call = lambda: lib.fd_decode_attn_paged(*a)  # noqa: E731
    check_rc(lib, call())
    t = timer.run([call], args.steps, args.warmup)
    check_rc(lib, call())
    # parity sample: the shortest and the longest sequence, through the
    # oracle's own block-table gather on a pool of just their pages
    picks = [int(min(range(B), key=lambda i: lens[i])), int(max(range(B), key=lambda i: lens[i]))]
    npg = [(int(lens[i]) + c.page - 1) // c.page for i in picks]
    pages = torch.cat([c.block_table[i, :m].long() for i, m in zip(picks, npg)])
    kp, vpool = _host(c.k_pool[pages]), _host(c.v_pool[pages])
    table = torch.zeros((2, max(npg)), dtype=torch.int32)
    table[0, :npg[0]] = torch.arange(npg[0], dtype=torch.int32)
    table[1, :npg[1]] = torch.arange(npg[0], npg[0] + npg[1], dtype=torch.int32)
    qs, os_, ls_ = _host(c.q[picks]), _host(out[picks]), _host(lse[picks])
    plens = [int(lens[i]) for i in picks]

    def check():
        import numpy as np
        from oracle import paged as opg
        f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
        ref, lref = opg.paged_attention(f(qs), kp.float().numpy(), vpool.float().numpy(),
                                        table.numpy(), np.array(plens), c.page, c.scale)
        return _errs(np, f(os_), f(ls_), ref, lref, 2e-3, 2 * Hq)
    PARITY_SAMPLES.append((f"config3 paged ragged bf16 (sequences of {plens[0]} and "
                           f"{plens[1]} positions, all heads)", check))
    total_len = int(sum(lens))
    nbytes = (2 * total_len * Hkv * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
              + 4 * int(sum((L + c.page - 1) // c.page for L in lens)))
    return dict(workload=f"paged ragged GQA decode bf16, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, "
                         f"page={c.page}, lens U[{cfg['len_lo']},{cfg['len_hi']}] "
                         f"(sum {total_len}, max {max_len}), chunk={c.chunk}",
                us_per_step=round(t["ms"] * 1e3, 2), p10_us=round(t["p10"] * 1e3, 2),
                p90_us=round(t["p90"] * 1e3, 2), bytes=nbytes,
                gbs=round(gbs(nbytes, t["ms"]), 1),
                pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1))


def variant_paged_multi(torch, fd, W, args, timer):
    """Four new tokens per sequence over the paged workload's cache (16
    sequences of U[1024, 131072] positions, pages of 16, chunk 1024 and 2048
    beside it): G*M = 16 query rows per kv-head on the matrix-core kernel;
    under M_8 the same with eight tokens (32 rows, the wave pair)."""
    cfg = W.CONFIGS[3]

    def measure(M):
        c = W.paged_case(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["len_lo"], cfg["len_hi"],
                         page=cfg["page"], chunk=cfg["chunk"], seed=cfg["seed"], device="cuda:0",
                         M=M)
        B, _, Hq, d = c.q.shape
        Hkv = c.k_pool.shape[1]
        lens = c.meta["lens"]
        max_len = int(max(lens))
        lib = fd.lib()
        out = torch.empty((B, M, Hq, d), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device="cuda:0")
        st = C.c_void_p(torch.cuda.current_stream().cuda_stream)

        def timed(chunk):
            wsn = fd.workspace_bytes("fd_decode_attn_multi_paged", B=B, M=M, Hq=Hq, Hkv=Hkv, d=d,
                                     page=c.page, max_pages=c.block_table.shape[1],
                                     max_seq_len=max_len, chunk=chunk)
            ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
            size = C.c_size_t(wsn)
            a = (fd.FD_BF16, vp(c.q), vp(c.k_pool), vp(c.v_pool), vp(c.block_table),
                 vp(c.seq_lens), vp(out), vp(lse), B, M, Hq, Hkv, d, c.page,
                 c.block_table.shape[1], c.k_pool.shape[0], max_len, c.scale, chunk, vp(ws),
                 C.byref(size), st)
            call = lambda: lib.fd_decode_attn_multi_paged(*a)  # noqa: E731
            check_rc(lib, call())
            return timer.run([call], args.steps, args.warmup)

        t = timed(c.chunk)
        t2 = timed(2 * c.chunk)
        total_len = int(sum(lens))
        nbytes = (2 * total_len * Hkv * d * 2 + B * M * Hq * d * 2 + B * M * Hq * (d + 1) * 4
                  + 4 * int(sum((L + c.page - 1) // c.page for L in lens)))
        res = dict(workload=f"paged ragged multi-row decode bf16, M={M} tokens, B={B}, Hq={Hq}, "
                            f"Hkv={Hkv}, d={d}, page={c.page}, lens U[{cfg['len_lo']},"
                            f"{cfg['len_hi']}] (sum {total_len}), chunk={c.chunk}",
                   us_per_step=round(t["ms"] * 1e3, 2), p10_us=round(t["p10"] * 1e3, 2),
                   p90_us=round(t["p90"] * 1e3, 2), bytes=nbytes,
                   gbs=round(gbs(nbytes, t["ms"]), 1),
                   pct_of_peak=round(100 * gbs(nbytes, t["ms"]) / PEAK_GBS, 1),
                   us_per_step_chunk2048=round(t2["ms"] * 1e3, 2),
                   pct_of_peak_chunk2048=round(100 * gbs(nbytes, t2["ms"]) / PEAK_GBS, 1))
        del c, out, lse
        torch.cuda.empty_cache()
        return res

    res = measure(4)
    res["M_8"] = measure(8)
    return res


def variant_unified(torch, fd, W, args, timer):
    c = W.config_case(4, device="cuda:0")
    B, Hq, d = c.q.shape
    Hkv, L = c.k.shape[1], c.k.shape[2]
    nc = (L + c.chunk - 1) // c.chunk
    ks = [c.k] + [c.k.clone() for _ in range(args.copies - 1)]
    vs = [c.v] + [c.v.clone() for _ in range(args.copies - 1)]
    lib = fd.lib()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    flags = torch.zeros((B, Hq, nc), dtype=torch.uint8, device="cuda:0")
    wsn = fd.workspace_bytes("fd_decode_attn_unified_max", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d,
                             chunk=c.chunk)
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def mk_u(k, v):
        a = (fd.FD_BF16, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
             c.chunk, c.phi, c.margin_hi, c.margin_lo, vp(flags), vp(ws), C.byref(size), st)
        return lambda: lib.fd_decode_attn_unified_max(*a)

    def mk_d(k, v):
        a = (fd.FD_BF16, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
             c.chunk, vp(ws), C.byref(size), st)
        return lambda: lib.fd_decode_attn(*a)

    uni = [mk_u(k, v) for k, v in zip(ks, vs)]
    den = [mk_d(k, v) for k, v in zip(ks, vs)]
    check_rc(lib, uni[0]())
    torch.cuda.synchronize()
    planted_b = sorted({b for b, _, _ in c.overflow_heads})
    sample_rows(torch, f"config4 fixed maximum bf16 (sequences {planted_b} holding the heads "
                f"planted above phi, all heads)", c.q[planted_b], c.k[planted_b],
                c.v[planted_b], out[planted_b], lse[planted_b], c.scale)
    flagged_heads = int(flags.sum())
    G = Hq // Hkv
    unit_flags = flags.view(B, Hkv, G, nc).amax(2)
    fallback_units = int(unit_flags.sum())
    check_rc(lib, den[0]())
    t = interleaved(timer, {"u": uni, "d": den}, args.steps, args.warmup)
    t_u, t_d = t["u"], t["d"]
    nbytes = 2 * B * Hkv * L * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
    return dict(workload=f"fixed-maximum decode bf16, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, L={L}, "
                         f"chunk={c.chunk}, phi={c.phi}, margins +{c.margin_hi}/-{c.margin_lo}, "
                         f"{len(c.overflow_heads)} heads planted above phi",
                us_per_step=round(t_u["ms"] * 1e3, 2), p10_us=round(t_u["p10"] * 1e3, 2),
                p90_us=round(t_u["p90"] * 1e3, 2), bytes=nbytes,
                gbs=round(gbs(nbytes, t_u["ms"]), 1),
                pct_of_peak=round(100 * gbs(nbytes, t_u["ms"]) / PEAK_GBS, 1),
                flagged_head_chunks=flagged_heads, fallback_chunks=fallback_units,
                fallback_reread_bytes=0,
                dense_same_data_us_per_step=round(t_d["ms"] * 1e3, 2),
                dense_over_unified=round(t_d["ms"] / t_u["ms"], 3))


def selected_variants(spec):
    """Variant names of a comma-separated --variants value, checked."""
    want = [x for x in spec.split(",") if x]
    unknown = [x for x in want if x not in VARIANTS]
    if unknown:
        sys.exit(f"unknown variants {unknown}; choose from {list(VARIANTS)}")
    return want


def _ffd_override(args):
    if args.ffd_deltas is None:
        return {}
    return dict(deltas=tuple(float(x) for x in args.ffd_deltas.split(",") if x))


def selection_quality(torch, q, k, scale, mask, delta):
    """How FFD's candidate set C compares with the exact top-delta set
    T = { j : s_j >= max_j s_j - delta } of the true scores s_j = scale q.K_j
    (FFD digest, section 3), per query head: recall |C & T| / |T|, and the
    share of the softmax mass that C keeps, sum_{j in C} e^{s_j - m} over
    sum_j e^{s_j - m}.  q [B,Hq,d], k [B,Hkv,L,d], mask int32 [B,Hq,ceil(L/32)]
    (bit j%32 of word j/32).  Plain fp32 products outside any timed region: a
    diagnostic of the selection, not part of the decode path."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    shifts = torch.arange(32, device=mask.device, dtype=torch.int32)
    rec, mass = [], []
    for b in range(B):
        qt = q[b].float().reshape(Hkv, G, d).transpose(1, 2).contiguous()   # [Hkv, d, G]
        s = (torch.matmul(k[b].float(), qt) * scale).transpose(1, 2).reshape(Hq, L)
        m = s.amax(-1, keepdim=True)
        top = s >= m - delta
        cand = ((mask[b].unsqueeze(-1) >> shifts) & 1).reshape(Hq, -1)[:, :L].bool()
        rec.append((cand & top).sum(-1).double() / top.sum(-1).double())
        w = torch.exp((s - m).double())
        mass.append((w * cand).sum(-1) / w.sum(-1))
    rec, mass = torch.cat(rec), torch.cat(mass)
    return dict(recall_exact_topdelta_mean=round(float(rec.mean()), 5),
                recall_exact_topdelta_min=round(float(rec.min()), 5),
                softmax_mass_kept_mean=round(float(mass.mean()), 6),
                softmax_mass_kept_min=round(float(mass.min()), 6))


def _ffd_sample(torch, name, c, pack, delta, out, lse, b, groups):
    """Register an FFD parity sample: sequence b, kv-groups `groups`, every
    query head of them (the oracle packs the bf16 keys itself and must
    produce the same bytes as the GPU packer)."""
    G = c.q.shape[1] // c.v.shape[1]
    q = _host(c.q[b])
    ks = {g: _host(c.k[b, g]) for g in groups}
    vs = {g: _host(c.v[b, g]) for g in groups}
    gp = {g: {key: _host(val[b, g]) for key, val in pack.items()} for g in groups}
    o, l_ = _host(out[b]), _host(lse[b])

    def check():
        import numpy as np
        from oracle import ffd as offd
        eo = el = 0.0
        same_pack = True
        for g in groups:
            ref = offd.pack_keys(ks[g].to(torch.float64).numpy().astype(np.float32))
            got = {"codes": gp[g]["codes"].numpy().view(np.uint32),
                   "zs": gp[g]["zs"].numpy().view(np.float16),
                   "res": gp[g]["res"].numpy(), "rs": gp[g]["rs"].numpy().view(np.float16)}
            same_pack &= all(np.array_equal(got[key].view(np.uint8), ref[key].view(np.uint8))
                             for key in ref)
            K2, Kh = offd.dequant(ref, q.shape[-1])
            V = vs[g].to(torch.float64).numpy()
            for h in range(g * G, (g + 1) * G):
                r = offd.ffd_row(q[h].to(torch.float64).numpy(), K2, Kh, V, c.scale, delta,
                                 c.n_sink, c.n_local)
                eo = max(eo, float(np.abs(o[h].to(torch.float64).numpy() - r["out"]).max()))
                el = max(el, abs(float(l_[h]) - r["lse"]))
        return dict(rows=len(groups) * G, max_abs_err_out=eo, max_abs_err_lse=el, tol=2e-3,
                    within_tol=bool(eo <= 2e-3 and el <= 2e-3), pack_bytes_equal=bool(same_pack),
                    note="positions within 1e-4 of the top-delta threshold may fall either way "
                         "(the tests bound their effect exactly); none of these rows needs it "
                         "when within_tol is true")
    PARITY_SAMPLES.append((name, check))


def _ffd_counts(np, mask, B, Hkv, G, L):
    m = mask.cpu().numpy().view(np.uint32).reshape(B, Hkv, G, -1)
    per_head = np.unpackbits(m.view(np.uint8), axis=-1).sum(-1)   # [B,Hkv,G]
    n_union = int(np.unpackbits(np.bitwise_or.reduce(m, axis=2).view(np.uint8), axis=-1).sum())
    return per_head, n_union


def _ffd_bytes(B, Hkv, L, d, Hq, n_anchor, n_union):
    return (B * Hkv * L * (d // 4 + d // 32 * 4) + n_union * (d + d // 32 * 2 + 2 * d)
            + B * Hkv * n_anchor * (d // 4 + d // 32 * 6 + d)
            + B * Hq * d * 2 + B * Hq * (d + 1) * 4)


def _ffd_variant(torch, fd, W, args, timer, cfg_id, label):
    """FFD sparse decode against dense attention on the same data: both
    timed first, interleaved (median of 3 rounds, each with its own warm-up);
    the candidate-set statistics and the selection quality (GPU-side
    diagnostics) only afterwards, outside every timed region.  Dense reads
    the bf16 keys, FFD the packed ones."""
    import numpy as np
    c = W.config_case(cfg_id, device="cuda:0", **_ffd_override(args))
    B, Hq, d = c.q.shape
    Hkv, L = c.v.shape[1], c.v.shape[2]
    G = Hq // Hkv
    lib = fd.lib()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    packs = [fd.ffd_pack(c.k)]
    torch.cuda.synchronize()
    pack_ms = (time.perf_counter() - t0) * 1e3
    packs += [{k: v.clone() for k, v in packs[0].items()} for _ in range(args.copies - 1)]
    ks = [c.k] + [c.k.clone() for _ in range(args.copies - 1)]
    vs = [c.v] + [c.v.clone() for _ in range(args.copies - 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda:0")
    wsn = max(fd.workspace_bytes("fd_ffd_sparse_decode", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d,
                                 chunk=c.chunk),
              fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, chunk=512))
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda:0")
    size = C.c_size_t(wsn)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def mk_d(k, v):
        a = (fd.FD_BF16, vp(c.q), vp(k), vp(v), vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale,
             512, vp(ws), C.byref(size), st)
        return lambda: lib.fd_decode_attn(*a)

    def mk_f(p, v, delta):
        a = (vp(c.q), vp(p["codes"]), vp(p["zs"]), vp(p["res"]), vp(p["rs"]), vp(v),
             vp(out), vp(lse), B, Hq, Hkv, L, d, c.scale, float(delta), c.n_sink,
             c.n_local, c.chunk, None, None, vp(ws), C.byref(size), st)
        return lambda: lib.fd_ffd_sparse_decode(*a)

    groups = {"dense": [mk_d(k, v) for k, v in zip(ks, vs)]}
    for delta in c.deltas:
        groups[f"delta_{delta:g}"] = [mk_f(p, v, delta) for p, v in zip(packs, vs)]
    for calls in groups.values():
        check_rc(lib, calls[0]())
    t = interleaved(timer, groups, args.steps, args.warmup)

    # diagnostics, outside the timed region
    dense_bytes = 2 * B * Hkv * L * d * 2 + B * Hq * d * 2 + B * Hq * (d + 1) * 4
    res = dict(workload=f"{label}, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, L={L}, chunk={c.chunk}, "
                        f"sinks={c.n_sink}, local={c.n_local}",
               pack_ms_whole_cache=round(pack_ms, 2),
               dense_us_per_step=round(t["dense"]["ms"] * 1e3, 2),
               dense_gbs=round(gbs(dense_bytes, t["dense"]["ms"]), 1),
               dense_bf16_bytes=dense_bytes)
    n_anchor = min(L, c.n_sink + c.n_local)
    for delta in c.deltas:
        key = f"delta_{delta:g}"
        _, _, mask, _ = fd.ffd_sparse_decode(c.q, packs[0], c.v, delta, c.n_sink, c.n_local,
                                             chunk=c.chunk, want_mask=True, out=out, lse=lse)
        per_head, n_union = _ffd_counts(np, mask, B, Hkv, G, L)
        quality = selection_quality(torch, c.q, c.k, c.scale, mask, delta)
        del mask
        _ffd_sample(torch, f"config{cfg_id} {label} delta {delta:g} (sequence 0, kv-groups 0 "
                    f"and {Hkv - 1})", c, packs[0], delta, out, lse, 0, (0, Hkv - 1))
        nbytes = _ffd_bytes(B, Hkv, L, d, Hq, n_anchor, n_union)
        ms = t[key]["ms"]
        res[key] = dict(us_per_step=round(ms * 1e3, 2), p10_us=round(t[key]["p10"] * 1e3, 2),
                        p90_us=round(t[key]["p90"] * 1e3, 2), bytes=int(nbytes),
                        gbs=round(gbs(nbytes, ms), 1),
                        pct_of_peak=round(100 * gbs(nbytes, ms) / PEAK_GBS, 1),
                        speedup_vs_dense=round(t["dense"]["ms"] / ms, 3),
                        kept_per_head=round(float(per_head.mean()) / L, 4),
                        kept_group_union=round(n_union / (B * Hkv * L), 4), **quality)
    return res


def variant_ffd(torch, fd, W, args, timer):
    return _ffd_variant(torch, fd, W, args, timer, 5, "FFD sparse decode (iid scores)")


def variant_ffd_peaked(torch, fd, W, args, timer):
    """Sharp queries whose heads of a group attend alike (per-head sparsity
    at the levels the FFD digest reports)."""
    return _ffd_variant(torch, fd, W, args, timer, 6,
                        "FFD vs dense on peaked queries (scale 5, group-shared 0.95)")


def main():
    args = parse_args()
    want = selected_variants(args.variants)
    _ffd_override(args)   # rejects a malformed --ffd-deltas before any GPU work
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU split is a design note, not a built path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import long_context_decode_fd_amd as fd
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    timer = Timer(torch, args.settle_ms)
    case, h = dense_headline(torch, fd, W, args, timer)
    line = {
        "metric": METRIC,
        "value": round(h["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["t_full"]["ms"], 5),
        "us_per_step": round(h["t_full"]["ms"] * 1e3, 2),
        "us_per_step_p10_p50_p90": [round(h["t_full"][k] * 1e3, 2) for k in ("p10", "p50", "p90")],
        "spread_method": "per-step mean of each window of 4 back-to-back steps (second pass)",
        "pct_of_peak": round(100 * h["value"] / PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded iid N(0,1) q/K/V rounded to bf16 (no model weights)",
        "config": h["workload"],
        "roofline": {
            "bound": "hbm",
            "kernel": "partial_kernel (split-KV chunk partials)",
            "achieved": round(h["achieved"], 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(h["achieved"] / PEAK_GBS, 4),
            "traffic": read_traffic(),
            "algorithmic_bytes_per_launch": h["part_bytes"],
            "launch_us_mean": round(h["t_part"]["ms"] * 1e3, 2),
        },
    }
    if not args.no_variants:
        fns = dict(config1=variant_config1, dense_b1=variant_dense_b1,
                   dense_128k=variant_dense_128k,
                   groups=variant_groups, paged=variant_paged,
                   paged_multi=variant_paged_multi,
                   unified_max=variant_unified, ffd=variant_ffd, ffd_peaked=variant_ffd_peaked,
                   multi_row=variant_multi, append=variant_append)
        line["variants"] = {name: fns[name](torch, fd, W, args, timer)
                            for name in VARIANTS if name in want}
    if not args.no_cpu_baseline:
        # the CPU leg: the oracle timed on the host cores, then the sampled
        # rows of every timed workload compared with it
        line["cpu_baseline"] = cpu_baseline(torch, case, args.cpu_seconds)
        line["parity_sample"] = {name: fn() for name, fn in PARITY_SAMPLES}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
