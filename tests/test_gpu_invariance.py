"""GPU invariances and special cases (decode and prefill through the C ABI).

* Segment order in the table and the physical placement of blocks do not
  change the result (zero-copy reuse, "LazyAttention" §1/§3 problem statement).
* With an identity cos/sin table (cos = 1, sin = 0) the kernels compute plain
  softmax attention over the gathered keys: compared with the oracle with RoPE
  switched off, this checks gather, GQA and softmax independently of rotation.
* Long positions (up to 2^17, the paper's 128K consistency study, App. C.4 /
  Table 7) in fp32 mode keep the 1e-5 bar.
"""
import numpy as np
import pytest
import torch

from oracle import run_decode, run_prefill
from position_agnostic_kv_lazy_amd import lazy_attn_validate_table
from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
from workloads import Segment, build_workload

from gpu_util import Device, assert_lse, assert_parity, config, log

pytestmark = pytest.mark.gpu


def _tiny(kind="decode", dtype="bf16", requests=None, Hq=8, Hkv=2, seed=21, q_pos_override=None):
    if requests is None:
        requests = ([[("doc", 0), ("doc", 1), ("doc", 2), ("priv", 5)],
                     [("doc", 3), ("doc", 0), ("doc", 1)]] if kind == "decode" else
                    [[("doc", 0), ("doc", 1), ("new", 40)], [("doc", 3), ("doc", 2), ("new", 70)]])
    return build_workload(name="inv", kind=kind, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=128, block_size=16, rope_base=5e5, doc_lens=[48, 37, 64, 20],
                          requests=requests, seed=seed, q_pos_override=q_pos_override)


def _with_segments(w, requests):
    import copy
    w2 = copy.copy(w)
    w2.requests = requests
    return w2


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_segment_order_does_not_matter(kind):
    w = _tiny(kind)
    dev = Device(w)
    o1, l1, _ = dev.run(w)
    rev = _with_segments(w, [list(reversed(segs)) for segs in w.requests])
    o2, l2, _ = dev.run(rev)
    assert_parity(o2, o1, "bf16", f"{kind} reversed segments vs table order")


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_block_relocation_does_not_matter(kind):
    """Copy every block to a new physical id (second half of a doubled pool)."""
    w = _tiny(kind)
    nb = w.num_blocks
    w2 = _with_segments(w, [[Segment(s.start, s.n_tokens, s.blocks + nb, s.is_new) for s in segs]
                            for segs in w.requests])
    w2.k_pool = np.concatenate([w.k_pool, w.k_pool])
    w2.v_pool = np.concatenate([w.v_pool, w.v_pool])
    o1, _, _ = Device(w).run(w)
    o2, _, _ = Device(w2).run(w2)
    np.testing.assert_array_equal(o1, o2)  # identical inputs, identical schedule


def _run_identity_table(w):
    k, v = upload_pool(w.k_pool, w.v_pool, "cuda")
    db = prepare(w, k, v)
    ident = np.zeros_like(db.cos_sin.cpu().numpy())
    ident[:, : w.head_dim // 2] = 1.0  # cos = 1, sin = 0 at every position
    db.cos_sin = torch.from_numpy(ident).cuda()
    db.run()
    torch.cuda.synchronize()
    return db.out_f32(), db.lse.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_identity_table_is_plain_attention(kind, dtype):
    w = _tiny(kind, dtype)
    log(f"identity table {kind} {dtype}")
    out, lse = _run_identity_table(w)
    if kind == "decode":
        ref = run_decode(w, rotate=False)
        for r in range(w.batch):
            assert_parity(out[r], ref[r][0], dtype, f"identity decode req {r}")
            assert_lse(lse[r], ref[r][1], dtype, f"identity decode req {r}")
    else:
        ref = run_prefill(w, rotate=False)
        for r in range(w.batch):
            a, b = int(w.cu_q[r]), int(w.cu_q[r + 1])
            assert_parity(out[a:b], ref[r][0], dtype, f"identity prefill req {r}")
            assert_lse(lse[a:b], ref[r][1], dtype, f"identity prefill req {r}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_positions_near_2_pow_17(dtype):
    """Documents placed at ~128K positions; query at 131000."""
    base = 130000
    reqs = [[("doc", 0, base - 5000), ("doc", 1, base), ("doc", 2, 3), ("priv", 7, base + 900)]]
    w = _tiny("decode", dtype, requests=reqs, q_pos_override=[131000])
    log(f"positions near 2^17 ({dtype})")
    out, lse, _ = Device(w).run(w)
    ref = run_decode(w)
    assert_parity(out[0], ref[0][0], dtype, "long positions")
    assert_lse(lse[0], ref[0][1], dtype, "long positions")


def test_config4_fp32_mode_sampled():
    w = config(4, dtype="f32", scale_down=4)
    log("config 4 shapes (scaled 1/4), fp32 mode")
    out, lse, _ = Device(w).run(w)
    reqs = [0, w.batch - 1]
    res = run_decode(w, requests=reqs)
    for r in reqs:
        assert_parity(out[r], res[r][0], "f32", f"cfg4-f32 req {r}")


def test_config5_fp32_mode_sampled():
    m = config(5, dtype="f32", scale_down=8)
    log("config 5 shapes (scaled 1/8), fp32 mode, both halves on one pool")
    dev = Device(m.prefill)
    od, _, _ = dev.run(m.decode)
    op, _, _ = dev.run(m.prefill)
    rd = run_decode(m.decode, requests=[0, 5])
    for r in (0, 5):
        assert_parity(od[r], rd[r][0], "f32", f"cfg5-f32 decode req {r}")
    rows = {0: np.array([0, 1, 63, 64, 127])}
    rp = run_prefill(m.prefill, requests=[0], rows=rows)
    assert_parity(op[rows[0]], rp[0][0], "f32", "cfg5-f32 prefill req 0")


def test_stale_hip_error_is_not_reported():
    """An unrelated failed HIP call left on the thread does not fail our launch."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch and the library share
    w = _tiny("decode", "bf16")
    k, v = upload_pool(w.k_pool, w.v_pool, "cuda")
    db = prepare(w, k, v)
    torch.cuda.synchronize()
    n = ctypes.c_int(0)
    assert hip.hipGetDeviceCount(ctypes.byref(n)) == 0
    assert hip.hipSetDevice(n.value + 7) != 0  # invalid ordinal: a host-side error only
    db.run()  # must not raise
    torch.cuda.synchronize()
    ref = run_decode(w)
    assert_parity(db.out_f32()[0], ref[0][0], "bf16", "after a stale HIP error")


def test_positions_at_the_24_bit_limit():
    """Keys and queries up to position 2^24 - 1, the largest the block word encodes (fp32 mode)."""
    import time
    top = (1 << 24) - 1
    dreq = [[("doc", 0, top - 700), ("doc", 1, 5), ("doc", 2, top - 64)]]
    wd = build_workload(name="lim", kind="decode", dtype="f32", num_q_heads=4, num_kv_heads=2,
                        head_dim=64, block_size=16, rope_base=1e4, doc_lens=[48, 37, 64],
                        requests=dreq, seed=3, q_pos_override=[top])
    preq = [[("doc", 0, top - 700), ("new", 40, top - 39)]]
    wp = build_workload(name="lim", kind="prefill", dtype="f32", num_q_heads=4, num_kv_heads=2,
                        head_dim=64, block_size=16, rope_base=1e4, doc_lens=[48, 37, 64],
                        requests=preq, seed=3)
    assert wd.table_rows() == 1 << 24 and wp.table_rows() == 1 << 24
    t0 = time.time()
    from position_agnostic_kv_lazy_amd import lazy_attn_rope_table
    table = lazy_attn_rope_table(wd.rope_base, wd.head_dim, 1 << 24)
    log(f"2^24-row table built in {time.time() - t0:.1f} s")
    od, ld, _ = Device(wd).run(wd, table=table)
    rd = run_decode(wd)
    assert_parity(od[0], rd[0][0], "f32", "decode at 2^24 - 1")
    assert_lse(ld[0], rd[0][1], "f32", "decode at 2^24 - 1")
    op, lp, _ = Device(wp).run(wp, table=table)
    rp = run_prefill(wp)
    assert_parity(op, rp[0][0], "f32", "prefill ending at 2^24 - 1")
    assert_lse(lp, rp[0][1], "f32", "prefill ending at 2^24 - 1")
