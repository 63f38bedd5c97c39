"""Both decode entry points driven from a plain C99 program on the GPU
(tests/c/abi_gpu_decode.c): hipMalloc'd buffers, the null stream, no Python
or torch in the process that launches the kernels.  The inputs are written
here from a seeded synthetic batch (device layouts: V tiles dim-major), the
outputs read back and compared with the fp64 oracle."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import run_decode
from workloads import build_workload

from gpu_util import assert_parity, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "position_agnostic_kv_lazy_amd")


def test_c_program_runs_both_decodes(tmp_path):
    import position_agnostic_kv_lazy_amd as la
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    w = build_workload(name="c_abi", kind="decode", dtype="bf16", num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, rope_base=5e5, doc_lens=[40, 33, 64],
                       requests=[[("doc", 0), ("doc", 1), ("doc", 2)],
                                 [("doc", 2), ("doc", 0, 500), ("priv", 5)],
                                 [("doc", 1, 17), ("doc", 2, 90)]], seed=31)
    rows = int(w.table_rows())
    p = la.make_params(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                       num_blocks=int(w.num_blocks), dtype="bf16", scale=w.scale, max_pos=rows)
    words, rbs, maxb = la.lazy_attn_pack_segments(p, w.requests)
    info, blob = la.lazy_attn_plan_shared_decode(p, w.requests)
    cs = la.lazy_attn_rope_table(w.rope_base, 128, rows)
    d = tmp_path
    np.ascontiguousarray(w.q, np.uint16).tofile(d / "q.bin")
    np.ascontiguousarray(w.k_pool, np.uint16).tofile(d / "k.bin")
    np.ascontiguousarray(np.asarray(w.v_pool, np.uint16).transpose(0, 1, 3, 2)).tofile(d / "v.bin")
    np.ascontiguousarray(words, np.uint64).tofile(d / "words.bin")
    np.ascontiguousarray(rbs, np.int32).tofile(d / "rbs.bin")
    np.ascontiguousarray(w.q_pos, np.int32).tofile(d / "qpos.bin")
    np.ascontiguousarray(cs, np.float32).tofile(d / "cs.bin")
    blob.tofile(d / "plan.bin")
    scale_bits = int(np.float32(w.scale).view(np.uint32))
    meta = [8, 2, 128, 16, int(w.num_blocks), rows, w.batch, int(maxb), len(words), scale_bits,
            info.n_items, info.n_members, info.n_words, info.members_per_item,
            info.max_item_blocks, info.plan_bytes]
    (d / "meta.txt").write_text(" ".join(str(x) for x in meta))
    exe = d / "abi_gpu_decode"
    b = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_gpu_decode.c"), "-o", str(exe),
                        "-L", LIBDIR, "-llazyattn", "-L", "/opt/rocm/lib", "-lamdhip64",
                        f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"],
                       capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stdout + b.stderr
    log("C caller: lazy_attn_decode and lazy_attn_decode_shared on the null stream")
    r = subprocess.run([str(exe), str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
    ref = run_decode(w)
    want = np.stack([ref[i][0] for i in range(w.batch)])
    for name in ("out_per_request.bin", "out_shared.bin"):
        bits = np.fromfile(d / name, dtype=np.uint16).reshape(w.batch, 8, 128)
        got = (bits.astype(np.uint32) << 16).view(np.float32)
        assert_parity(got, want, "bf16", f"C caller {name}")
