"""Prefill parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every row; the full-size configurations (the launch the
benchmark times) compare a seeded sample of rows per request, chosen to hit
q-tile boundaries and the causal tail.
"""
import numpy as np
import pytest

from oracle import run_prefill
from workloads import build_workload

from gpu_util import Device, assert_lse, assert_parity, config, log

pytestmark = pytest.mark.gpu


def _tiny(dtype="bf16", Hq=8, Hkv=2, requests=None, doc_lens=(40, 33, 16, 70, 5), seed=6,
          poison=False):
    if requests is None:
        requests = [[("doc", 0), ("doc", 1), ("new", 37)],
                    [("doc", 3), ("doc", 0), ("doc", 1), ("new", 200)],
                    [("doc", 4), ("new", 1)],
                    [("new", 20, 100), ("doc", 2, 0), ("doc", 1, 40)]]
    return build_workload(name="tiny", kind="prefill", dtype=dtype, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=128, block_size=16, rope_base=5e5,
                          doc_lens=list(doc_lens), requests=requests, seed=seed, poison_tail=poison)


def _check_rows(w, out, lse, rows_of, what):
    res = run_prefill(w, requests=list(rows_of), rows=rows_of)
    for r, rows in rows_of.items():
        a = int(w.cu_q[r])
        o_ref, l_ref = res[r]
        assert_parity(out[a + np.asarray(rows)], o_ref, w.dtype, f"{what} req {r}")
        assert_lse(lse[a + np.asarray(rows)], l_ref, w.dtype, f"{what} req {r}")


def _all_rows(w):
    return {r: np.arange(w.q_len(r)) for r in range(w.batch)}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1), (32, 8), (32, 2)])
def test_tiny_groups(dtype, Hq, Hkv):
    """Ragged q lengths (1..200), partial blocks, new segment listed first."""
    w = _tiny(dtype=dtype, Hq=Hq, Hkv=Hkv)
    log(f"tiny prefill {dtype} Hq={Hq} Hkv={Hkv}")
    out, lse, _ = Device(w).run(w)
    _check_rows(w, out, lse, _all_rows(w), "tiny")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_poisoned_tail_slots(dtype):
    w = _tiny(dtype=dtype, poison=True)
    log(f"poisoned tails prefill {dtype}")
    out, lse, _ = Device(w).run(w)
    _check_rows(w, out, lse, _all_rows(w), "poison")


def test_new_tokens_only():
    """No cached document: plain causal attention over the new tokens."""
    w = _tiny(requests=[[("new", 150)], [("new", 16, 5000)]])
    out, lse, _ = Device(w).run(w)
    _check_rows(w, out, lse, _all_rows(w), "new-only")


def test_shift_invariance_gpu():
    reqs = [[("doc", 0), ("doc", 3), ("new", 45)]]
    c = 9000
    reqs_c = [[("doc", 0, c), ("doc", 3, c + 40), ("new", 45, c + 110)]]
    w0 = _tiny(requests=reqs)
    w1 = _tiny(requests=reqs_c)
    dev = Device(w0)
    o0, _, _ = dev.run(w0)
    o1, _, _ = dev.run(w1)
    assert_parity(o1, o0, "bf16", "shifted vs unshifted")


def _sample_rows(n, rng, extra=()):
    base = {0, 1, 31, 32, 33, 127, 128, n // 2, n - 2, n - 1, *extra}
    base |= set(rng.choice(n, size=min(n, 12), replace=False).tolist())
    return np.array(sorted(x for x in base if 0 <= x < n))


def test_config3_every_request():
    """The benchmark's prefill batch: every request, seeded sample of rows each."""
    w = config(3)
    log("config 3 full size (8 x 10240 cached + 512 new), all requests")
    out, lse, _ = Device(w).run(w)
    rng = np.random.default_rng(33)
    rows = {r: _sample_rows(w.q_len(r), rng) for r in range(w.batch)}
    _check_rows(w, out, lse, rows, "cfg3")


def test_config3_fp32_mode():
    w = config(3, dtype="f32", scale_down=4)
    log("config 3 shapes, fp32 mode")
    out, lse, _ = Device(w).run(w)
    rng = np.random.default_rng(34)
    rows = {r: _sample_rows(w.q_len(r), rng) for r in range(w.batch)}
    _check_rows(w, out, lse, rows, "cfg3-f32")


def test_config5_prefill_sampled():
    m = config(5)
    log("config 5 prefill half (4 x 10240 cached + 1024 new)")
    out, lse, _ = Device(m.prefill).run(m.prefill)
    rng = np.random.default_rng(35)
    rows = {r: _sample_rows(m.prefill.q_len(r), rng, extra=(511, 512, 1023)) for r in range(4)}
    _check_rows(m.prefill, out, lse, rows, "cfg5-pre")


def test_first_tile_far_below_zero():
    """A row whose first key tile scores far below 0 (< -128 in log2 units).

    The kernel's first softmax reference for that row then lies far below the
    initial 0; the accumulators must not be rescaled by exp2(-delta), which
    overflows.  Identity cos/sin table, so the oracle is plain attention.
    """
    from workloads import f32_to_bf16_bits
    w = _tiny(requests=[[("doc", 0), ("doc", 1), ("new", 40)]], doc_lens=(64, 37))
    blocks = np.asarray(w.requests[0][0].blocks)
    spike = np.zeros(w.head_dim, np.float32)
    spike[0] = 40.0
    w.k_pool[blocks] = f32_to_bf16_bits(spike)  # every key of doc 0 = 40 e_0
    qf = w.values_f32(w.q).copy()
    qf[..., 0] = -40.0  # q . k = -1600 on doc 0: about -204 in log2 units after scaling
    w.q = f32_to_bf16_bits(qf)
    ident = np.zeros((w.table_rows(), w.head_dim), np.float32)
    ident[:, : w.head_dim // 2] = 1.0
    out, lse, _ = Device(w).run(w, table=ident)
    ref = run_prefill(w, rotate=False)
    a, b = int(w.cu_q[0]), int(w.cu_q[1])
    assert_parity(out[a:b], ref[0][0], "bf16", "far-negative first tile")
    assert_lse(lse[a:b], ref[0][1], "bf16", "far-negative first tile")
