#!/usr/bin/env python3
"""Benchmark of the lazy-RoPE paged attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--no-extra] [--no-cpu]

A step is one call of the hot path on one batch with every input already in
HBM: by default the Llama-3-8B-shaped decode layer (64 requests, 10 Zipf(1.0)
documents of 512 tokens + a 64-token question each, 32 q / 8 kv heads,
head_dim 128, bf16).  `value` is the logical K+V bytes the step must read
(4096 B per key across the 8 kv heads) divided by the step time, in GB/s.
The same run also measures (unless --no-extra) the prefill, long-context
decode and mixed decode+prefill workloads, each against its roofline, and
(unless --no-cpu) the fp64 CPU oracle on a bounded sample of the headline
workload.  Prints ONE JSON line.

W defaults to 500 untimed launches: this GPU reaches its steady clocks only
after some tens of milliseconds of back-to-back work, and a decode launch
takes 0.16 ms, so a 10-launch warm-up would time the ramp.
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
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
WARM_S = 0.25               # minimum warm-up (seconds of launches) for the extra workloads
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
KERNEL_SRC = {
    "decode": os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "csrc", "decode_bf16.hip"),
    "prefill": os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "csrc", "prefill_bf16.hip"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(kind):
    with open(KERNEL_SRC[kind], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kind, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kind}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != src_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(run, steps, warmup, stream, flush=None, min_warm_s=0.0):
    """Warm up, then time exactly `steps` back-to-back launches by wall clock, and
    `steps` more with per-launch HIP events.

    The GPU raises its clocks only after some tens of milliseconds of sustained
    work (a 0.17 ms decode launch runs about 10 % slower for its first ~150
    back-to-back launches), so steady-state figures need enough warm-up:
    `warmup` launches, continued until at least `min_warm_s` seconds of them
    have run.
    """
    import torch
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_warm < min_warm_s:
        run()
        done += 1
        if done % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # Wall clock: exactly `steps` launches back to back, with nothing else on
    # the stream (per-launch event records would add their own gaps).
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush()
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-launch durations: the same `steps` launches again, each bracketed by
    # HIP events on the launch stream.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]  # ms
    return wall, float(np.mean(per)), float(np.median(per)), per


def make_flusher(nbytes=1 << 30):
    """Overwrite a buffer larger than L2 + Infinity Cache (1 GiB) to evict the pool."""
    import torch
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def flush():
        buf.fill_(1.0)
    return flush


def run_decode_workload(w, k, v, stream, steps, warmup, split_blocks=0, min_warm_s=WARM_S):
    from position_agnostic_kv_lazy_amd.prepare import prepare
    db = prepare(w, k, v, split_blocks=split_blocks)
    run = lambda: db.run(stream)  # noqa: E731
    wall, ev_mean, ev_med, per = time_launches(run, steps, warmup, stream, min_warm_s=min_warm_s)
    # right after the warm timing: the clocks are up, one warm-up launch suffices
    _, cold_mean, cold_med, _ = time_launches(run, max(5, steps // 2), 1, stream, make_flusher())
    nbytes = w.logical_kv_bytes()
    return {
        "logical_kv_bytes": nbytes,
        "wall_ms_per_step": 1e3 * wall / steps,
        "event_ms_mean": ev_mean,
        "event_ms_median": ev_med,
        "event_ms_p10": float(np.percentile(per, 10)),
        "event_ms_p90": float(np.percentile(per, 90)),
        "gbs_logical": nbytes / (ev_mean * 1e-3) / 1e9,
        "cold_event_ms_mean": cold_mean,
        "cold_gbs_logical": nbytes / (cold_mean * 1e-3) / 1e9,
        "workspace_bytes": 0 if db.workspace is None else int(db.workspace.numel()),
        "_db": db,
    }


def run_prefill_workload(w, k, v, stream, steps, warmup, min_warm_s=WARM_S):
    from position_agnostic_kv_lazy_amd.prepare import prepare
    db = prepare(w, k, v)
    run = lambda: db.run(stream)  # noqa: E731
    wall, ev_mean, ev_med, per = time_launches(run, steps, warmup, stream, min_warm_s=min_warm_s)
    flops = w.prefill_flops()
    return {
        "flops": flops,
        "wall_ms_per_step": 1e3 * wall / steps,
        "event_ms_mean": ev_mean,
        "event_ms_median": ev_med,
        "event_ms_p10": float(np.percentile(per, 10)),
        "event_ms_p90": float(np.percentile(per, 90)),
        "tflops": flops / (ev_mean * 1e-3) / 1e12,
        "_db": db,
    }


def roofline_hbm(nbytes, ms, kind, workload, split):
    """Decode roofline; `split` says whether the launch ran split groups (then a
    combine kernel follows the decode kernel and both are timed)."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = traffic_for(kind, workload)
    per_launch = {"algorithmic_bytes": nbytes, "avg_ms": round(ms, 5)}
    if traffic is not None:  # measured DRAM bytes at the same rate: the real HBM load
        per_launch["dram_gbs"] = round(traffic / (ms * 1e-3) / 1e9, 1)
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "decode_bf16_kernel + decode_combine_kernel" if split else "decode_bf16_kernel",
            "per_launch": per_launch}


def roofline_mfma(flops, ms, kind, workload):
    tfs = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "traffic": traffic_for(kind, workload), "kernel": "prefill_bf16_kernel",
            "per_launch": {"algorithmic_flops": flops, "avg_ms": round(ms, 5)}}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the headline workload.

    Requests (decode) or 16-row slices of new tokens (prefill) are run in turn
    until about budget_s seconds of single-threaded CPU work are done.
    """
    from threadpoolctl import threadpool_limits

    from oracle import run_decode, run_prefill
    t0 = time.perf_counter()
    work = 0
    units = 0
    with threadpool_limits(limits=1):
        if w.kind == "decode":
            keys = w.keys_per_request()
            while time.perf_counter() - t0 < budget_s or units < 2:
                r = units % w.batch
                run_decode(w, requests=[r])
                work += int(keys[r]) * w.num_kv_heads * w.head_dim * 2 * 2
                units += 1
            dt = time.perf_counter() - t0
            return {"value": round(work / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle", "cpu_model": _cpu_model(),
                    "visible_cores": len(os.sched_getaffinity(0)),
                    "sample": f"{units} decode requests (cycling over the {w.batch}-request "
                              f"batch), fp64 NumPy, BLAS limited to 1 thread, {dt:.1f} s"}
        cached = w.keys_per_request() - np.array([w.q_len(r) for r in range(w.batch)])
        while time.perf_counter() - t0 < budget_s or units < 1:
            r = units % w.batch
            rows = np.arange(16 * (units // w.batch) % w.q_len(r), w.q_len(r))[:16]
            run_prefill(w, requests=[r], rows={r: rows})
            work += int(sum(4 * w.head_dim * w.num_q_heads * (int(cached[r]) + int(j) + 1)
                            for j in rows))
            units += 1
        dt = time.perf_counter() - t0
        return {"value": round(work / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                "kind": "oracle", "cpu_model": _cpu_model(),
                "visible_cores": len(os.sched_getaffinity(0)),
                "sample": f"{units} slices of 16 new-token rows, fp64 NumPy, BLAS limited to "
                          f"1 thread, {dt:.1f} s"}


def _clean(res):
    return {kk: (round(vv, 5) if isinstance(vv, float) else vv)
            for kk, vv in res.items() if not kk.startswith("_")}


def _extra_no_sharing(stream, steps):
    """Control for the shared-document mix: configuration 2's shapes with every
    request reading its own documents, so logical bytes = unique bytes = what
    DRAM must deliver."""
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_no_sharing_decode
    try:
        log("no-sharing control (64 requests x 10 private documents)")
        w = make_no_sharing_decode()
        k, v = upload_pool(w.k_pool, w.v_pool)
        res = run_decode_workload(w, k, v, stream, steps, 3)
        out = _clean(res)
        out["frac_of_hbm_peak"] = round(res["gbs_logical"] / HBM_PEAK_GBS, 4)
        out["cold_frac_of_hbm_peak"] = round(res["cold_gbs_logical"] / HBM_PEAK_GBS, 4)
        return {w.name: out}
    except Exception as e:  # reported, never hidden
        return {"no_sharing_control": {"error": repr(e)}}


def _extra_achievable(stream):
    """Reference rates measured on the same GPU in the same run: a plain 1 GiB
    device copy (torch copy_) and a plain bf16 GEMM (torch.matmul, 8192^3)."""
    import torch
    try:
        log("achievable references: 1 GiB copy, 8192^3 bf16 GEMM")
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        _, copy_ms, _, _ = time_launches(lambda: dst.copy_(src), 10, 3, stream,
                                         min_warm_s=WARM_S)
        del src, dst
        n = 8192
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        _, gemm_ms, _, _ = time_launches(lambda: torch.matmul(a, b, out=c), 10, 3, stream,
                                         min_warm_s=WARM_S)
        del a, b, c
        torch.cuda.empty_cache()
        return {"achievable_references": {
            "copy_1gib_gbs_moved": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_8192_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "note": "plain copy reads + writes 1 GiB; GEMM through torch.matmul (hipBLASLt)"}}
    except Exception as e:  # reported, never hidden
        return {"achievable_references": {"error": repr(e)}}


def _extra_prefill(stream, steps):
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_config
    try:
        log("prefill (Llama-3-8B shapes, 8 requests x 10240 cached + 512 new)")
        w3 = make_config(3)
        k3, v3 = upload_pool(w3.k_pool, w3.v_pool)
        r3 = run_prefill_workload(w3, k3, v3, stream, steps, 3)
        out = _clean(r3)
        out["roofline"] = roofline_mfma(r3["flops"], r3["event_ms_mean"], "prefill", w3.name)
        return {w3.name: out}
    except Exception as e:  # reported, never hidden
        return {"llama3_8b_prefill": {"error": repr(e)}}


def _extra_long_decode(stream, steps):
    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_config
    try:
        log("long-context decode (16 requests x 64K keys)")
        w4 = make_config(4)
        k4, v4 = upload_pool(w4.k_pool, w4.v_pool)
        r4 = run_decode_workload(w4, k4, v4, stream, steps, 3)
        out = _clean(r4)
        out["roofline"] = roofline_hbm(r4["logical_kv_bytes"], r4["event_ms_mean"], "decode",
                                       w4.name, r4["workspace_bytes"] > 0)
        return {w4.name: out}
    except Exception as e:  # reported, never hidden
        return {"long_decode": {"error": repr(e)}}


def _extra_mixed(stream, steps):
    """Config 5: one decode launch and one prefill launch on one shared pool."""
    import torch

    from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
    from workloads import make_config
    try:
        log("mixed step: 128 decode + 4 prefill requests on one pool")
        m5 = make_config(5)
        k5, v5 = upload_pool(m5.prefill.k_pool, m5.prefill.v_pool)
        dd = prepare(m5.decode, k5, v5)
        dp = prepare(m5.prefill, k5, v5)
        s2 = torch.cuda.Stream()

        def pair_two_streams():
            ev = torch.cuda.Event()
            ev.record(stream)
            s2.wait_event(ev)
            dp.run(s2)
            dd.run(stream)
            e2 = torch.cuda.Event()
            e2.record(s2)
            stream.wait_event(e2)

        def pair_serial():
            dp.run(stream)
            dd.run(stream)

        _, p2, _, _ = time_launches(pair_two_streams, steps, 3, stream, min_warm_s=WARM_S)
        _, p1, _, _ = time_launches(pair_serial, steps, 3, stream, min_warm_s=WARM_S)
        _, dm, _, _ = time_launches(lambda: dd.run(stream), steps, 3, stream, min_warm_s=WARM_S)
        _, fm, _, _ = time_launches(lambda: dp.run(stream), steps, 3, stream, min_warm_s=WARM_S)
        nb = m5.decode.logical_kv_bytes()
        fl = m5.prefill.prefill_flops()
        return {"mixed_step": {
            "pair_serial_event_ms_mean": round(p1, 5),
            "pair_two_streams_event_ms_mean": round(p2, 5),
            "decode_event_ms_mean": round(dm, 5),
            "prefill_event_ms_mean": round(fm, 5),
            "decode_gbs_logical": round(nb / (dm * 1e-3) / 1e9, 1),
            "prefill_tflops": round(fl / (fm * 1e-3) / 1e12, 1),
            "decode_logical_kv_bytes": nb, "prefill_flops": fl,
        }}
    except Exception as e:
        return {"mixed_step": {"error": repr(e)}}


def _extra_rotation_ablation(w, k, v, stream, steps, pf_out):
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
    All three outputs are compared with the position-free path's output.
    """
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

    def decode(wx, kd, vd):
        db = prepare(wx, kd, vd, pool_mode="doc_local", max_pos=rows)
        _, ms, _, _ = time_launches(lambda: db.run(stream), steps, 3, stream, min_warm_s=WARM_S)
        torch.cuda.synchronize()
        diff = float((db.out.view(torch.bfloat16).float() - pos_free).abs().max())
        return db, ms, diff

    nbytes = w.logical_kv_bytes()
    # ---- document-local pool
    slots, idx = segment_slots(w, "index")
    kt, vt = gather(slots)
    kd, vd = torch.zeros_like(k), torch.zeros_like(v)
    p_w = params_for(w, int(k.shape[0]), rows)
    run_w = store(p_w, kt, vt, slots, idx, kd, vd)
    _, wms, _, _ = time_launches(run_w, max(3, steps // 4), 1, stream, min_warm_s=WARM_S)
    moved = 4 * len(slots) * Hkv * D * 2
    _, dms, diff = decode(w, kd, vd)
    res["doc_local"] = {
        "decode_event_ms_mean": round(dms, 5),
        "decode_gbs_logical": round(nbytes / (dms * 1e-3) / 1e9, 1),
        "write_tokens": int(len(slots)), "write_event_ms_mean": round(wms, 5),
        "write_gbs": round(moved / (wms * 1e-3) / 1e9, 1),
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
    run_m = store(p_m, kt, vt, dst, pos, km, vm)
    _, mms, _, _ = time_launches(run_m, max(3, steps // 4), 1, stream, min_warm_s=WARM_S)
    moved = 4 * len(dst) * Hkv * D * 2
    import copy
    wm = copy.copy(w)
    wm.requests = reqs
    _, rms, diff = decode(wm, km, vm)
    res["materialised"] = {
        "decode_event_ms_mean": round(rms, 5),
        "decode_gbs_logical": round(nbytes / (rms * 1e-3) / 1e9, 1),
        "copy_tokens": int(len(dst)), "copy_event_ms_mean": round(mms, 5),
        "copy_gbs": round(moved / (mms * 1e-3) / 1e9, 1),
        "copy_plus_decode_ms": round(mms + rms, 5),
        "pool_bytes": int(km.numel() * 2 * 2), "shared_pool_bytes": int(k.numel() * 2 * 2),
        "max_abs_diff_vs_position_free": diff}
    del kt, vt, km, vm
    torch.cuda.empty_cache()

    # ---- ALiBi (score-space positional method, no rotation) on the position-free pool
    db = prepare(w, k, v, pos_encoding="alibi", max_pos=rows)
    _, ams, _, _ = time_launches(lambda: db.run(stream), steps, 3, stream, min_warm_s=WARM_S)
    res["alibi"] = {"decode_event_ms_mean": round(ams, 5),
                    "decode_gbs_logical": round(nbytes / (ams * 1e-3) / 1e9, 1)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4],
                    help="headline workload: 2 decode (default), 3 prefill, 4 long decode")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (to scale PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from position_agnostic_kv_lazy_amd.prepare import upload_pool
    from workloads import make_config

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

    log(f"generating config {args.config}")
    w = make_config(args.config)
    k, v = upload_pool(w.k_pool, w.v_pool)
    wl_name = w.name
    config = {"workload": wl_name, "batch": w.batch, "q_heads": w.num_q_heads,
              "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
              "docs": "Zipf document mix, shared physical blocks"}
    ablation = None
    if w.kind == "decode":
        log("timing headline decode")
        main_res = run_decode_workload(w, k, v, stream, args.steps, args.warmup, args.split_blocks,
                                       min_warm_s=0.0)
        if not args.no_extra:
            log("rotation ablation: doc-local pool and materialised copies")
            try:
                ablation = _extra_rotation_ablation(w, k, v, stream, max(5, args.steps // 2),
                                                    main_res["_db"].out.view(torch.bfloat16))
                ablation["position_free_decode_event_ms_mean"] = round(main_res["event_ms_mean"],
                                                                       5)
            except Exception as e:  # reported, never hidden
                ablation = {"error": repr(e)}
            torch.cuda.empty_cache()
        ms = main_res["wall_ms_per_step"]
        value, unit = main_res["logical_kv_bytes"] / (ms * 1e-3) / 1e9, "GB/s"
        config["keys_per_request"] = int(w.keys_per_request()[0])
        roof = roofline_hbm(main_res["logical_kv_bytes"], main_res["event_ms_mean"], "decode",
                            wl_name, main_res["workspace_bytes"] > 0)
    else:
        log("timing headline prefill")
        main_res = run_prefill_workload(w, k, v, stream, args.steps, args.warmup, min_warm_s=0.0)
        ms = main_res["wall_ms_per_step"]
        value, unit = main_res["flops"] / (ms * 1e-3) / 1e12, "TFLOP/s"
        config["new_tokens_per_request"] = int(w.q_len(0))
        config["cached_keys_per_request"] = int(w.keys_per_request()[0] - w.q_len(0))
        roof = roofline_mfma(main_res["flops"], main_res["event_ms_mean"], "prefill", wl_name)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
    }
    extra = {wl_name: _clean(main_res)}
    if ablation is not None:
        extra["rotation_ablation"] = ablation
    del main_res, k, v
    torch.cuda.empty_cache()

    if not args.no_extra:
        steps2 = max(5, args.steps // 2)
        if args.config != 3:
            extra.update(_extra_prefill(stream, steps2))
            torch.cuda.empty_cache()
        if args.config != 4:
            extra.update(_extra_long_decode(stream, steps2))
            torch.cuda.empty_cache()
        extra.update(_extra_mixed(stream, steps2))
        torch.cuda.empty_cache()
        if args.config == 2:
            extra.update(_extra_no_sharing(stream, steps2))
            torch.cuda.empty_cache()
        extra.update(_extra_achievable(stream))
    result["extra"] = extra

    if not args.no_cpu:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
