#!/usr/bin/env python3
"""Benchmark of the lazy-RoPE paged attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--legs L]
                    [--no-extra] [--no-cpu]

A step is one call of the hot path on one batch with every input already in
HBM: by default the Llama-3-8B-shaped decode layer (64 requests, 10 Zipf(1.0)
documents of 512 tokens + a 64-token question each, 32 q / 8 kv heads,
head_dim 128, bf16).  `value` is the logical K+V bytes the step must read
(4096 B per key across the 8 kv heads) divided by the step time, in GB/s.

`roofline` is the HBM roofline of the decode kernel on the bytes HBM actually
delivers per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE, recorded in
profiles/traffic.json for the kernel source it was measured on) divided by
the launch time from HIP events: shared documents are served from L2 and the
Infinity Cache, so the logical bytes overstate what HBM moves.  The same run
also measures (unless --no-extra) the prefill, long-context decode, mixed
decode+prefill and no-sharing control workloads, each against its roofline,
and (unless --no-cpu) the fp64 CPU oracle over the host cores on the whole
headline batch and on sampled prefill rows -- whose results also check the
outputs of the timed launches.  Prints ONE JSON line.

Warm-up: every leg, the headline included, runs at least W launches and at
least WARM_S seconds of launches before timing (this GPU reaches its steady
clocks only after some tens of milliseconds of back-to-back work); the
launches actually run are reported per leg.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn KV GB/s (% HBM peak) + prefill TFLOPS (% MFMA peak), 1 GPU"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
WARM_S = 0.25                # minimum warm-up (seconds of launches) for every leg
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
KERNEL_SRC = {
    "decode": os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "csrc", "decode_bf16.hip"),
    "decode_shared": os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "csrc",
                                  "decode_shared_bf16.hip"),
    "prefill": os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "csrc", "prefill_bf16.hip"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
LEGS = ("headline", "other_decode", "ablation", "prefill", "long_decode", "mixed", "no_sharing",
        "references")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(kind):
    with open(KERNEL_SRC[kind], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kind, workload, plan_sha=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel
    is unchanged and, for a record taken with a shared-decode plan, the plan
    blob is the same (the plan decides the chunks and partials)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kind}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != src_hash(kind):
        return None
    if "plan_sha256_16" in rec and rec["plan_sha256_16"] != plan_sha:
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- CPU oracle
# The oracle runs in worker processes forked before this process touches the
# GPU; the workloads they read are module globals set before the fork.  No
# worker ever makes a GPU call.
_ORACLE_W = {}


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)  # one BLAS thread per worker process


def _oracle_decode_one(args):
    key, r = args
    from oracle import run_decode
    out, lse = run_decode(_ORACLE_W[key], requests=[r])[r]
    return r, out, lse


def _oracle_prefill_rows(args):
    key, r, rows = args
    from oracle import run_prefill
    out, lse = run_prefill(_ORACLE_W[key], requests=[r], rows={r: np.asarray(rows)})[r]
    return r, rows, out, lse


class OraclePool:
    """Process pool over the visible host cores, forked before any GPU call."""

    def __init__(self):
        import multiprocessing as mp
        self.cores = len(os.sched_getaffinity(0))
        self.pool = mp.get_context("fork").Pool(self.cores, initializer=_oracle_worker_init)

    def decode(self, key, requests):
        t0 = time.perf_counter()
        res = self.pool.map(_oracle_decode_one, [(key, r) for r in requests], chunksize=1)
        return {r: (o, l) for r, o, l in res}, time.perf_counter() - t0

    def prefill(self, key, rows_by_req):
        t0 = time.perf_counter()
        jobs = [(key, r, rows[i:i + 8]) for r, rows in rows_by_req.items()
                for i in range(0, len(rows), 8)]
        res = self.pool.map(_oracle_prefill_rows, jobs, chunksize=1)
        out = {}
        for r, rows, o, l in res:
            out.setdefault(r, []).append((rows, o, l))
        return out, time.perf_counter() - t0

    def close(self):
        self.pool.terminate()
        self.pool.join()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _errors(gpu, ref):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.max(np.abs(g - r))), float(np.linalg.norm(g - r) / np.linalg.norm(r))


def _parity(gpu_rows, ref_rows, what):
    max_abs, rel = _errors(np.concatenate([g.reshape(-1) for g in gpu_rows]),
                           np.concatenate([r.reshape(-1) for r in ref_rows]))
    ok = bool(np.all(np.isfinite(np.concatenate([g.reshape(-1) for g in gpu_rows])))
              and max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2)
    return {"checked": what, "max_abs": float(f"{max_abs:.4g}"), "rel_l2": float(f"{rel:.4g}"),
            "tolerance": {"max_abs": BF16_MAX_ABS, "rel_l2": BF16_REL_L2}, "pass": ok}


# --------------------------------------------------------------------- timing
def time_launches(run, steps, warmup, stream, flush=None, min_warm_s=WARM_S):
    """Warm up (at least `warmup` launches and `min_warm_s` seconds of them), then
    time exactly `steps` back-to-back launches by wall clock, and `steps` more
    with per-launch HIP events on the launch stream (optionally each after
    `flush()`).  Returns a dict of the figures and the warm-up launches run."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_warm < min_warm_s:
        run()
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    wall = None
    if flush is None:
        # Wall clock: exactly `steps` launches back to back, with nothing else
        # on the stream (per-launch event records would add their own gaps).
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])  # ms
    return {"wall_s": wall, "mean": float(per.mean()), "median": float(np.median(per)),
            "p10": float(np.percentile(per, 10)), "p90": float(np.percentile(per, 90)),
            "warmup_launches": done}


def make_flushers(nbytes=1 << 30):
    """Two ways to evict the pool from L2 and the Infinity Cache between cold
    repetitions: a read-only sweep of a 1 GiB buffer (leaves no dirty lines),
    and a 1 GiB fill (whose dirty lines are written back while the next
    launch runs)."""
    import torch
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def read_sweep():
        torch.sum(buf, dim=0, out=sink)

    def write_fill():
        buf.fill_(1.0)
    return read_sweep, write_fill


def _ms(x):
    return round(x, 5)


MAX_ITEM_BLOCKS = 0  # shared-decode chunk length (0: the library default); set by --max-item-blocks


def run_decode_workload(w, k, v, stream, steps, warmup, split_blocks=0, cold=True, shared=False):
    """Time one decode workload: lazy_attn_decode_shared (shared=True) or lazy_attn_decode."""
    from position_agnostic_kv_lazy_amd.prepare import prepare
    db = prepare(w, k, v, split_blocks=split_blocks, shared=shared,
                 max_item_blocks=MAX_ITEM_BLOCKS)
    run = lambda: db.run(stream)  # noqa: E731
    t = time_launches(run, steps, warmup, stream)
    nbytes = w.logical_kv_bytes()
    res = {
        "logical_kv_bytes": nbytes,
        "unique_kv_bytes": w.unique_kv_bytes(),
        "warmup_launches": t["warmup_launches"],
        "wall_ms_per_step": 1e3 * t["wall_s"] / steps,
        "event_ms_mean": t["mean"], "event_ms_median": t["median"],
        "event_ms_p10": t["p10"], "event_ms_p90": t["p90"],
        "gbs_logical": nbytes / (t["mean"] * 1e-3) / 1e9,
        "workspace_bytes": 0 if db.workspace is None else int(db.workspace.numel()),
        "decode_kernel": "shared" if shared else "per_request",
        "_db": db,
    }
    if shared:
        res["plan"] = {"items": db.plan_info.n_items, "partials": db.plan_info.n_members,
                       "distinct_chunk_blocks": db.plan_info.n_words,
                       "chunk_blocks": db.plan_info.max_item_blocks,
                       "sha256_16": hashlib.sha256(db.host_plan.tobytes()).hexdigest()[:16]}
    if cold:
        read_sweep, write_fill = make_flushers()
        n = max(5, steps // 2)
        # right after the warm timing: the clocks are up, one warm-up launch suffices
        c = time_launches(run, n, 1, stream, read_sweep, min_warm_s=0.0)
        cw = time_launches(run, n, 1, stream, write_fill, min_warm_s=0.0)
        res.update({
            "cold_event_ms_mean": c["mean"], "cold_event_ms_median": c["median"],
            "cold_gbs_logical": nbytes / (c["mean"] * 1e-3) / 1e9,
            "cold_after_write_flush_event_ms_mean": cw["mean"],
            "cold_after_write_flush_gbs_logical": nbytes / (cw["mean"] * 1e-3) / 1e9,
            "cold_flush": "1 GiB read-only sweep before each launch (primary); the "
                          "write-flush figure fills 1 GiB instead, whose dirty lines are "
                          "written back during the timed launch",
        })
        del read_sweep, write_fill
    return res


def run_prefill_workload(w, k, v, stream, steps, warmup):
    from position_agnostic_kv_lazy_amd.prepare import prepare
    db = prepare(w, k, v)
    run = lambda: db.run(stream)  # noqa: E731
    t = time_launches(run, steps, warmup, stream)
    flops = w.prefill_flops()
    return {
        "flops": flops,
        "warmup_launches": t["warmup_launches"],
        "wall_ms_per_step": 1e3 * t["wall_s"] / steps,
        "event_ms_mean": t["mean"], "event_ms_median": t["median"],
        "event_ms_p10": t["p10"], "event_ms_p90": t["p90"],
        "tflops": flops / (t["mean"] * 1e-3) / 1e12,
        "_db": db,
    }


def roofline_hbm(res, kind, workload, split):
    """Decode HBM roofline on the bytes HBM delivers per launch (rocprofv3
    counters, same kernel source) over the launch time by HIP events."""
    ms = res["event_ms_mean"]
    if res.get("decode_kernel") == "shared":
        kind = "decode_shared"
        kern = "decode_shared_kernel + decode_shared_combine_kernel"
    else:
        kern = "decode_bf16_kernel + decode_combine_kernel" if split else "decode_bf16_kernel"
    traffic = traffic_for(kind, workload, res.get("plan", {}).get("sha256_16"))
    per_launch = {"algorithmic_bytes": res["logical_kv_bytes"],
                  "unique_bytes": res["unique_kv_bytes"],
                  "logical_gbs": round(res["logical_kv_bytes"] / (ms * 1e-3) / 1e9, 1),
                  "avg_ms": _ms(ms)}
    if traffic is None:
        # no counter record for this kernel source: the logical rate is all we have
        return {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": None, "traffic": None, "kernel": kern,
                "basis": "no HBM counter record for this kernel source", "per_launch": per_launch}
    gbs = traffic / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kern,
            "basis": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE, "
                     "profiles/traffic.json) / HIP-event launch time",
            "per_launch": per_launch}


def roofline_mfma(flops, ms, kind, workload):
    tfs = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "traffic": traffic_for(kind, workload), "kernel": "prefill_bf16_kernel",
            "per_launch": {"algorithmic_flops": flops, "avg_ms": _ms(ms)}}


def _clean(res):
    return {kk: (round(vv, 5) if isinstance(vv, float) else vv)
            for kk, vv in res.items() if not kk.startswith("_")}


# ---------------------------------------------------------------- extra legs
def _extra_no_sharing(stream, steps, warmup, shared):
    """Control for the shared-document mix: configuration 2's shapes with every
    request reading its own documents, so logical bytes = unique bytes = what
    DRAM must deliver.  Timed with both decode kernels: the headline's, and the
    other one (with nothing shared, the per-request decode is the natural
    choice)."""
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_no_sharing_decode
    out = {}
    try:
        log("no-sharing control (64 requests x 10 private documents)")
        w = make_no_sharing_decode()
        k, v = upload_pool(w.k_pool, w.v_pool)
        for kernel_shared in (shared, not shared):
            res = run_decode_workload(w, k, v, stream, steps, warmup, shared=kernel_shared)
            o = _clean(res)
            o["frac_of_hbm_peak"] = round(res["gbs_logical"] / HBM_PEAK_GBS, 4)
            o["cold_frac_of_hbm_peak"] = round(res["cold_gbs_logical"] / HBM_PEAK_GBS, 4)
            o["cold_after_write_flush_frac_of_hbm_peak"] = round(
                res["cold_after_write_flush_gbs_logical"] / HBM_PEAK_GBS, 4)
            name = w.name if kernel_shared == shared else (
                f"{w.name}_{res['decode_kernel']}_decode")
            out[name] = o
        return out
    except Exception as e:  # reported, never hidden
        out.setdefault("llama3_8b_decode_no_sharing", {"error": repr(e)})
        out["llama3_8b_decode_no_sharing_error"] = repr(e)
        return out


def _extra_achievable(stream, steps, warmup):
    """Reference rates measured on the same GPU in the same run: a plain 1 GiB
    device copy (torch copy_), a 1 GiB read-only sweep (torch sum) and a plain
    bf16 GEMM (torch.matmul, 8192^3)."""
    import torch
    try:
        log("achievable references: 1 GiB copy and read, 8192^3 bf16 GEMM")
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        copy = time_launches(lambda: dst.copy_(src), steps, warmup, stream)
        del dst
        srcf = src.view(torch.float32)
        sink = torch.empty((), dtype=torch.float32, device="cuda")
        rd = time_launches(lambda: torch.sum(srcf, dim=0, out=sink), steps, warmup, stream)
        del src, srcf
        n = 8192
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        gemm = time_launches(lambda: torch.matmul(a, b, out=c), steps, warmup, stream)
        del a, b, c
        torch.cuda.empty_cache()
        return {"achievable_references": {
            "copy_1gib_gbs_moved": round(2 * (1 << 30) / (copy["mean"] * 1e-3) / 1e9, 1),
            "read_1gib_gbs": round((1 << 30) / (rd["mean"] * 1e-3) / 1e9, 1),
            "gemm_bf16_8192_tflops": round(2 * n ** 3 / (gemm["mean"] * 1e-3) / 1e12, 1),
            "note": "plain copy reads + writes 1 GiB; read = torch.sum over 1 GiB; GEMM "
                    "through torch.matmul (hipBLASLt)"}}
    except Exception as e:  # reported, never hidden
        return {"achievable_references": {"error": repr(e)}}


def _extra_prefill(w3, stream, steps, warmup, oracle):
    """Config 3 prefill against the MFMA roofline; sampled rows of the timed
    launch's output are checked against the oracle, which is timed too."""
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    try:
        log("prefill (Llama-3-8B shapes, 8 requests x 10240 cached + 512 new)")
        k3, v3 = upload_pool(w3.k_pool, w3.v_pool)
        r3 = run_prefill_workload(w3, k3, v3, stream, steps, warmup)
        out = _clean(r3)
        out["roofline"] = roofline_mfma(r3["flops"], r3["event_ms_mean"], "prefill", w3.name)
        if oracle is not None:
            import torch
            torch.cuda.synchronize()
            got = r3["_db"].out_f32()
            # 64 rows per request: spread over the new tokens, first and last included
            rows = {r: np.unique(np.linspace(0, w3.q_len(r) - 1, 64).astype(np.int64))
                    for r in range(w3.batch)}
            log(f"oracle: prefill rows ({sum(len(x) for x in rows.values())}) on "
                f"{oracle.cores} cores")
            ref, dt = oracle.prefill("prefill", rows)
            g_rows, r_rows, flops = [], [], 0
            cached = w3.keys_per_request() - np.array([w3.q_len(r) for r in range(w3.batch)])
            for r, parts in ref.items():
                a = int(w3.cu_q[r])
                for rr, o, _ in parts:
                    g_rows.append(got[a + np.asarray(rr)])
                    r_rows.append(o)
                    flops += sum(4 * w3.head_dim * w3.num_q_heads * (int(cached[r]) + int(j) + 1)
                                 for j in rr)
            out["parity_vs_oracle"] = _parity(g_rows, r_rows,
                                              f"{sum(len(x) for x in rows.values())} sampled "
                                              f"new-token rows (all heads) of the timed launch")
            out["cpu_baseline"] = {
                "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.cores,
                "kind": "oracle", "cpu_model": _cpu_model(),
                "sample": f"{sum(len(x) for x in rows.values())} new-token rows (64 per "
                          f"request, all 32 heads) of the prefill batch, fp64 NumPy, "
                          f"{oracle.cores} worker processes x 1 BLAS thread, {dt:.1f} s"}
        return {w3.name: out}
    except Exception as e:  # reported, never hidden
        return {"llama3_8b_prefill": {"error": repr(e)}}


def _extra_long_decode(stream, steps, warmup, shared):
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_config
    try:
        log("long-context decode (16 requests x 64K keys)")
        w4 = make_config(4)
        k4, v4 = upload_pool(w4.k_pool, w4.v_pool)
        r4 = run_decode_workload(w4, k4, v4, stream, steps, warmup, shared=shared)
        out = _clean(r4)
        out["roofline"] = roofline_hbm(r4, "decode", w4.name, r4["workspace_bytes"] > 0)
        return {w4.name: out}
    except Exception as e:  # reported, never hidden
        return {"long_decode": {"error": repr(e)}}


def _extra_mixed(stream, steps, warmup, shared):
    """Config 5: one decode launch and one prefill launch on one shared pool."""
    import torch

    from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
    from workloads import make_config
    try:
        log("mixed step: 128 decode + 4 prefill requests on one pool")
        m5 = make_config(5)
        k5, v5 = upload_pool(m5.prefill.k_pool, m5.prefill.v_pool)
        dd = prepare(m5.decode, k5, v5, shared=shared, max_item_blocks=MAX_ITEM_BLOCKS)
        dp = prepare(m5.prefill, k5, v5)
        s2 = torch.cuda.Stream()

        def pair_two_streams():
            ev = torch.cuda.Event()
            ev.record(stream)
            s2.wait_event(ev)
            dd.run(s2)
            dp.run(stream)
            e2 = torch.cuda.Event()
            e2.record(s2)
            stream.wait_event(e2)

        def pair_serial():
            dd.run(stream)
            dp.run(stream)

        p2 = time_launches(pair_two_streams, steps, warmup, stream)
        p1 = time_launches(pair_serial, steps, warmup, stream)
        dm = time_launches(lambda: dd.run(stream), steps, warmup, stream)
        fm = time_launches(lambda: dp.run(stream), steps, warmup, stream)
        nb = m5.decode.logical_kv_bytes()
        fl = m5.prefill.prefill_flops()
        return {"mixed_step": {
            "pair_serial_event_ms_mean": _ms(p1["mean"]),
            "pair_two_streams_event_ms_mean": _ms(p2["mean"]),
            "decode_event_ms_mean": _ms(dm["mean"]),
            "prefill_event_ms_mean": _ms(fm["mean"]),
            "decode_gbs_logical": round(nb / (dm["mean"] * 1e-3) / 1e9, 1),
            "prefill_tflops": round(fl / (fm["mean"] * 1e-3) / 1e12, 1),
            "decode_logical_kv_bytes": nb, "decode_unique_kv_bytes": m5.decode.unique_kv_bytes(),
            "prefill_flops": fl, "decode_kernel": "shared" if shared else "per_request",
            "decode_plan": None if dd.host_plan is None else {
                "items": dd.plan_info.n_items, "partials": dd.plan_info.n_members,
                "chunk_blocks": dd.plan_info.max_item_blocks,
                "sha256_16": hashlib.sha256(dd.host_plan.tobytes()).hexdigest()[:16]},
            "warmup_launches": {"pair_two_streams": p2["warmup_launches"],
                                "pair_serial": p1["warmup_launches"],
                                "decode": dm["warmup_launches"],
                                "prefill": fm["warmup_launches"]},
        }}
    except Exception as e:
        return {"mixed_step": {"error": repr(e)}}


def _extra_rotation_ablation(w, k, v, stream, steps, warmup, pf_out):
    """Where deferred RoPE stands against the alternatives, on the headline decode batch.

    * doc_local: each distinct document written once with its keys pre-rotated
      by the in-document index (lazy_attn_store_kv), then decode in
      LA_POOL_DOC_LOCAL mode: q rotated once per segment, keys read as stored
      (the decode design of "LazyAttention" §3.2).
    * materialised: every request gets a private copy of its segments with keys
      rotated at their absolute positions (the re-encoding a position-aware
      cache needs for a document at a new offset), then the same decode with
      every segment start 0: no key rotation and one q rotation per request --
      the rotation-off baseline.  The copy itself is timed too: its bytes are
      the read-modify-write the shared position-free pool never does.
    * alibi: the same shared pool, no rotation at all.
    All outputs are compared with the position-free path's output.  Every
    leg uses the same warm-up rule as the headline.
    """
    import copy

    import torch

    from position_agnostic_kv_lazy_amd import binding as B
    from position_agnostic_kv_lazy_amd.prepare import params_for, prepare
    from workloads import private_copies, segment_slots
    res = {}
    BS, D, Hkv = w.block_size, w.head_dim, w.num_kv_heads
    rows = int(w.table_rows())
    cs = torch.from_numpy(B.lazy_attn_rope_table(w.rope_base, D, rows)).cuda()
    pos_free = pf_out.float()

    def gather(slots_np):
        sl = torch.from_numpy(slots_np).cuda()
        blk, slot = sl // BS, sl % BS
        return k[blk, :, slot, :].contiguous(), v[blk, :, :, slot].contiguous()

    def store(params, kt, vt, dst_np, pos_np, kd, vd):
        dst = torch.from_numpy(dst_np).cuda()
        pos = torch.from_numpy(pos_np).cuda()
        return lambda: B.lazy_attn_store_kv(params, kt, vt, len(dst_np), dst, pos, cs, kd, vd,
                                            stream)

    def decode(wx, kd, vd, shared=False):
        db = prepare(wx, kd, vd, pool_mode="doc_local", max_pos=rows, shared=shared)
        t = time_launches(lambda: db.run(stream), steps, warmup, stream)
        torch.cuda.synchronize()
        diff = float((db.out.view(torch.bfloat16).float() - pos_free).abs().max())
        return t, diff

    nbytes = w.logical_kv_bytes()
    # ---- document-local pool
    slots, idx = segment_slots(w, "index")
    kt, vt = gather(slots)
    kd, vd = torch.zeros_like(k), torch.zeros_like(v)
    p_w = params_for(w, int(k.shape[0]), rows)
    tw = time_launches(store(p_w, kt, vt, slots, idx, kd, vd), max(3, steps // 4), 1, stream)
    moved = 4 * len(slots) * Hkv * D * 2
    td, diff = decode(w, kd, vd)
    res["doc_local"] = {
        "decode_event_ms_mean": _ms(td["mean"]),
        "decode_gbs_logical": round(nbytes / (td["mean"] * 1e-3) / 1e9, 1),
        "decode_warmup_launches": td["warmup_launches"],
        "write_tokens": int(len(slots)), "write_event_ms_mean": _ms(tw["mean"]),
        "write_gbs": round(moved / (tw["mean"] * 1e-3) / 1e9, 1),
        "max_abs_diff_vs_position_free": diff}
    ts, diff = decode(w, kd, vd, shared=True)
    res["doc_local_shared_decode"] = {
        "decode_event_ms_mean": _ms(ts["mean"]),
        "decode_gbs_logical": round(nbytes / (ts["mean"] * 1e-3) / 1e9, 1),
        "decode_warmup_launches": ts["warmup_launches"],
        "max_abs_diff_vs_position_free": diff}
    del kt, vt, kd, vd
    torch.cuda.empty_cache()

    # ---- materialised per-request copies (rotation-off baseline)
    reqs, src, dst, pos = private_copies(w)
    kt, vt = gather(src)
    nb_m = int(dst.max()) // BS + 1
    km = torch.zeros((nb_m,) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    vm = torch.zeros((nb_m,) + tuple(v.shape[1:]), dtype=v.dtype, device=v.device)
    p_m = params_for(w, nb_m, rows)
    tm = time_launches(store(p_m, kt, vt, dst, pos, km, vm), max(3, steps // 4), 1, stream)
    moved = 4 * len(dst) * Hkv * D * 2
    wm = copy.copy(w)
    wm.requests = reqs
    tr, diff = decode(wm, km, vm)
    res["materialised"] = {
        "decode_event_ms_mean": _ms(tr["mean"]),
        "decode_gbs_logical": round(nbytes / (tr["mean"] * 1e-3) / 1e9, 1),
        "decode_warmup_launches": tr["warmup_launches"],
        "copy_tokens": int(len(dst)), "copy_event_ms_mean": _ms(tm["mean"]),
        "copy_gbs": round(moved / (tm["mean"] * 1e-3) / 1e9, 1),
        "copy_plus_decode_ms": _ms(tm["mean"] + tr["mean"]),
        "pool_bytes": int(km.numel() * 2 * 2), "shared_pool_bytes": int(k.numel() * 2 * 2),
        "max_abs_diff_vs_position_free": diff}
    del kt, vt, km, vm
    torch.cuda.empty_cache()

    # ---- ALiBi (score-space positional method, no rotation) on the position-free pool
    db = prepare(w, k, v, pos_encoding="alibi", max_pos=rows)
    ta = time_launches(lambda: db.run(stream), steps, warmup, stream)
    res["alibi"] = {"decode_event_ms_mean": _ms(ta["mean"]),
                    "decode_gbs_logical": round(nbytes / (ta["mean"] * 1e-3) / 1e9, 1),
                    "decode_warmup_launches": ta["warmup_launches"]}
    # the position-free pool under the per-request kernel, timed like the rows above
    db = prepare(w, k, v, max_pos=rows)
    tp = time_launches(lambda: db.run(stream), steps, warmup, stream)
    res["position_free"] = {"decode_event_ms_mean": _ms(tp["mean"]),
                            "decode_gbs_logical": round(nbytes / (tp["mean"] * 1e-3) / 1e9, 1),
                            "decode_warmup_launches": tp["warmup_launches"]}
    res["note"] = ("doc_local, materialised, alibi and position_free run the per-request kernel "
                   "(lazy_attn_decode); doc_local_shared runs the shared-segment kernel over the "
                   "document-local pool")
    return res


# ----------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4],
                    help="headline workload: 2 decode (default), 3 prefill, 4 long decode")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of " + ",".join(LEGS))
    ap.add_argument("--no-extra", action="store_true", help="headline leg only")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--decode", choices=["shared", "per_request"], default="shared",
                    help="decode kernel: lazy_attn_decode_shared (each shared segment read once "
                         "per launch) or lazy_attn_decode (one split per request)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (to scale PMC byte counters)")
    ap.add_argument("--max-item-blocks", type=int, default=0,
                    help="shared decode: blocks per work item (0 = library default)")
    args = ap.parse_args()
    global MAX_ITEM_BLOCKS
    MAX_ITEM_BLOCKS = args.max_item_blocks
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    legs = {"headline"} if args.no_extra else set(x for x in args.legs.split(",") if x)
    unknown = legs - set(LEGS)
    if unknown:
        print(f"unknown legs {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    from workloads import make_config

    # CPU side first: the workloads the oracle checks, then the oracle's worker
    # processes, forked before this process makes any GPU call.
    log(f"generating config {args.config}")
    w = make_config(args.config)
    w3 = None
    if "prefill" in legs and args.config != 3:
        w3 = make_config(3)
    oracle = None
    if not args.no_cpu:
        _ORACLE_W["headline"] = w
        _ORACLE_W["prefill"] = w3 if w3 is not None else w
        oracle = OraclePool()

    import torch

    from position_agnostic_kv_lazy_amd.prepare import upload_pool

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    wl_name = w.name
    config = {"workload": wl_name, "batch": w.batch, "q_heads": w.num_q_heads,
              "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
              "docs": "Zipf document mix, shared physical blocks"}
    steps2 = max(5, args.steps // 2)
    extra = {}
    ablation = None
    value = ms = roof = head_out = None
    unit = "GB/s" if w.kind == "decode" else "TFLOP/s"
    if "headline" not in legs:
        log("headline leg skipped (--legs): value and roofline are null")
    elif w.kind == "decode":
        k, v = upload_pool(w.k_pool, w.v_pool)
        shared = args.decode == "shared"
        log(f"timing headline decode ({args.decode})")
        main_res = run_decode_workload(w, k, v, stream, args.steps, args.warmup, args.split_blocks,
                                       shared=shared)
        torch.cuda.synchronize()
        head_out = main_res["_db"].out_f32()
        if "other_decode" in legs:
            other = "per_request" if shared else "shared"
            log(f"the other decode kernel ({other}) on the headline batch")
            try:
                o = run_decode_workload(w, k, v, stream, steps2, args.warmup, args.split_blocks,
                                        shared=not shared)
                torch.cuda.synchronize()
                diff = float(np.max(np.abs(o["_db"].out_f32() - head_out)))
                oc = _clean(o)
                oc["roofline"] = roofline_hbm(o, "decode", wl_name, o["workspace_bytes"] > 0)
                oc["max_abs_diff_vs_headline_kernel"] = diff
                extra[f"{wl_name}_{other}_decode"] = oc
                del o
            except Exception as e:  # reported, never hidden
                extra[f"{wl_name}_{other}_decode"] = {"error": repr(e)}
        if "ablation" in legs:
            log("rotation ablation: doc-local pool, materialised copies, ALiBi")
            try:
                ablation = _extra_rotation_ablation(w, k, v, stream, steps2, args.warmup,
                                                    main_res["_db"].out.view(torch.bfloat16))
            except Exception as e:  # reported, never hidden
                ablation = {"error": repr(e)}
            torch.cuda.empty_cache()
        ms = main_res["wall_ms_per_step"]
        value, unit = main_res["logical_kv_bytes"] / (ms * 1e-3) / 1e9, "GB/s"
        config["keys_per_request"] = int(w.keys_per_request()[0])
        roof = roofline_hbm(main_res, "decode", wl_name, main_res["workspace_bytes"] > 0)
    else:
        k, v = upload_pool(w.k_pool, w.v_pool)
        log("timing headline prefill")
        main_res = run_prefill_workload(w, k, v, stream, args.steps, args.warmup)
        head_out = None
        ms = main_res["wall_ms_per_step"]
        value, unit = main_res["flops"] / (ms * 1e-3) / 1e12, "TFLOP/s"
        config["new_tokens_per_request"] = int(w.q_len(0))
        config["cached_keys_per_request"] = int(w.keys_per_request()[0] - w.q_len(0))
        roof = roofline_mfma(main_res["flops"], main_res["event_ms_mean"], "prefill", wl_name)
    if "headline" in legs:
        extra[wl_name] = _clean(main_res)
        del main_res, k, v
    if ablation is not None:
        extra["rotation_ablation"] = ablation
    torch.cuda.empty_cache()

    if "prefill" in legs and args.config != 3:
        extra.update(_extra_prefill(w3, stream, steps2, args.warmup, oracle))
        torch.cuda.empty_cache()
    if "long_decode" in legs and args.config != 4:
        extra.update(_extra_long_decode(stream, steps2, args.warmup, args.decode == "shared"))
        torch.cuda.empty_cache()
    if "mixed" in legs:
        extra.update(_extra_mixed(stream, steps2, args.warmup, args.decode == "shared"))
        torch.cuda.empty_cache()
    if "no_sharing" in legs and args.config == 2:
        extra.update(_extra_no_sharing(stream, steps2, args.warmup, args.decode == "shared"))
        torch.cuda.empty_cache()
        ns = extra.get("llama3_8b_decode_no_sharing", {})
        other = "per_request" if args.decode == "shared" else "shared"
        ns2 = extra.get(f"llama3_8b_decode_no_sharing_{other}_decode", {})
        if "frac_of_hbm_peak" in ns and roof is not None:
            roof["controls"] = {
                "no_sharing_warm_frac": ns["frac_of_hbm_peak"],
                "no_sharing_cold_frac": ns["cold_frac_of_hbm_peak"],
                "no_sharing_cold_after_write_flush_frac":
                    ns["cold_after_write_flush_frac_of_hbm_peak"],
                "note": "configuration 2's shapes with no document shared: logical = unique "
                        "bytes = what HBM must deliver; cold = after a 1 GiB read-only sweep; "
                        f"the {other} fields time the other decode kernel on the same batch"}
            if "frac_of_hbm_peak" in ns2:
                roof["controls"].update({
                    f"no_sharing_{other}_warm_frac": ns2["frac_of_hbm_peak"],
                    f"no_sharing_{other}_cold_frac": ns2["cold_frac_of_hbm_peak"]})
    if "references" in legs:
        extra.update(_extra_achievable(stream, 10, 3))

    result = {
        "metric": METRIC,
        "value": None if value is None else round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if ms is None else round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
    }

    if oracle is not None:
        if w.kind == "decode" and head_out is not None:
            log(f"oracle: all {w.batch} headline requests on {oracle.cores} cores")
            ref, dt = oracle.decode("headline", range(w.batch))
            result["parity_vs_oracle"] = _parity(
                [head_out[r] for r in range(w.batch)], [ref[r][0] for r in range(w.batch)],
                f"all {w.batch} requests x {w.num_q_heads} heads of the timed headline launch")
            result["cpu_baseline"] = {
                "value": round(w.logical_kv_bytes() / dt / 1e9, 4), "unit": "GB/s",
                "cores": oracle.cores, "kind": "oracle", "cpu_model": _cpu_model(),
                "sample": f"the whole headline batch ({w.batch} requests, "
                          f"{int(w.keys_per_request().sum())} keys), fp64 NumPy, "
                          f"{oracle.cores} worker processes x 1 BLAS thread, {dt:.2f} s"}
        oracle.close()
    result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
