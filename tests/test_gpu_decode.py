"""Decode parity: the HIP path through the C ABI against the fp64 oracle.

bf16: max-abs 2e-2 and relative L2 5e-3 against the oracle on the exact bf16
inputs; fp32 test mode: max-abs 1e-5.  Full-size configurations check every
request where the oracle is cheap (config 2) and a seeded sample of requests
otherwise (configs 4 and 5), in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from oracle import run_decode
from workloads import build_workload

from gpu_util import Device, assert_lse, assert_parity, config, log

pytestmark = pytest.mark.gpu


def _check(w, res, reqs, what, outs, lses):
    for r in reqs:
        o, l = res[r]
        assert_parity(outs[r], o, w.dtype, f"{what} req {r}")
        assert_lse(lses[r], l, w.dtype, f"{what} req {r}")


def _tiny(dtype="bf16", Hq=8, Hkv=2, requests=None, doc_lens=(40, 33, 16, 70, 5), seed=5,
          q_pos_override=None, poison=False, D=128):
    if requests is None:
        requests = [[("doc", 0), ("doc", 1), ("priv", 3)],
                    [("doc", 1), ("doc", 2), ("doc", 0, 300)],
                    [("doc", 3), ("doc", 1), ("doc", 3, 500), ("priv", 1)],
                    [("doc", 4, 0)]]
    return build_workload(name="tiny", kind="decode", dtype=dtype, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, block_size=16, rope_base=5e5,
                          doc_lens=list(doc_lens), requests=requests, seed=seed,
                          q_pos_override=q_pos_override, poison_tail=poison)


def test_config1_fp32():
    w = config(1)
    log("config 1 (fp32, D=64)")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), [0], "cfg1", out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1), (32, 8), (32, 2)])
def test_tiny_groups(dtype, Hq, Hkv):
    """Partial tail blocks, 1-token segment, a document twice in one request."""
    w = _tiny(dtype=dtype, Hq=Hq, Hkv=Hkv)
    log(f"tiny decode {dtype} Hq={Hq} Hkv={Hkv}")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), range(w.batch), "tiny", out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_poisoned_tail_slots(dtype):
    """Unused slots of partial blocks hold NaN; they must never reach the output."""
    w = _tiny(dtype=dtype, poison=True)
    log(f"poisoned tails {dtype}")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), range(w.batch), "poison", out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_keys_after_query_and_self_key(dtype):
    """Negative relative offsets (keys past m) and the query's own position as a key."""
    reqs = [[("doc", 0), ("doc", 1), ("priv", 1)], [("doc", 2, 10), ("doc", 0, 700)]]
    # request 0: m = 40+33 (its own key at m is the 1-token private segment)
    # request 1: m = 200, document 0 sits at 700.. (after the query)
    w = _tiny(dtype=dtype, requests=reqs, q_pos_override=[73, 200])
    log(f"self key / keys after query {dtype}")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), range(w.batch), "offsets", out, lse)


def test_split_counts_agree():
    """Any split-group size gives the same result (bf16) and matches the oracle."""
    w = config(2, scale_down=8)
    dev = Device(w)
    ref = run_decode(w)
    outs = []
    for sb in (0, 1, 7, 64, 400):
        log(f"split_blocks={sb}")
        out, lse, db = dev.run(w, split_blocks=sb)
        _check(w, ref, range(w.batch), f"split{sb}", out, lse)
        outs.append(out)
    for o in outs[1:]:
        # identical inputs, different summation order: agree far inside tolerance
        assert np.max(np.abs(o - outs[0])) < 8e-3


def test_shift_invariance_gpu():
    """Moving every position by a constant leaves the GPU output unchanged (Fact 3.2)."""
    reqs = [[("doc", 0), ("doc", 1)], [("doc", 2), ("doc", 3)]]
    w0 = _tiny(requests=reqs)
    c = 4096
    reqs_c = [[("doc", 0, c), ("doc", 1, c + 40)], [("doc", 2, c), ("doc", 3, c + 16)]]
    w1 = _tiny(requests=reqs_c)
    dev = Device(w0)
    o0, _, _ = dev.run(w0)
    o1, _, _ = dev.run(w1)
    assert_parity(o1, o0, "bf16", "shifted vs unshifted")


def test_config2_full():
    w = config(2)
    log("config 2 full size")
    out, lse, db = Device(w).run(w)
    log(f"  split groups workspace={0 if db.workspace is None else db.workspace.numel()} bytes")
    _check(w, run_decode(w), range(w.batch), "cfg2", out, lse)


def test_config2_fp32_mode():
    w = config(2, dtype="f32", scale_down=4)
    log("config 2 shapes, fp32 mode")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w, requests=range(w.batch)), range(w.batch), "cfg2-f32", out, lse)


def test_config4_every_request():
    w = config(4)
    log("config 4 full size (64K context), all 16 requests")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), range(w.batch), "cfg4", out, lse)


def test_config2_fp32_mode_full_size():
    """fp32 test mode at the full Llama-3-8B decode shape (64 x 5,184 keys)."""
    w = config(2, dtype="f32")
    log("config 2 full size, fp32 mode")
    out, lse, _ = Device(w).run(w)
    _check(w, run_decode(w), range(w.batch), "cfg2-f32-full", out, lse)


def test_config5_decode_sampled():
    m = config(5)
    log("config 5 decode half, sampled requests")
    out, lse, _ = Device(m.decode, pool_of=m.prefill).run(m.decode)
    reqs = list(range(0, 128, 17))
    _check(m.decode, run_decode(m.decode, requests=reqs), reqs, "cfg5-dec", out, lse)
