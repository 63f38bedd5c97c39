"""The mixed serving step exactly as bench.py times it, against the oracle.

Configuration 5: 128 decode requests and 4 prefill requests over ONE device
pool (the same documents at different offsets within one batch, as the
problem statement of "LazyAttention" §3 asks), the decode launched first on a
second stream and the prefill on the current one, joined by events.  Both
halves are compared with the oracle on sampled requests and rows, for each
decode kernel.
"""
import numpy as np
import pytest
import torch

from oracle import run_decode, run_prefill
from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool

from gpu_util import assert_lse, assert_parity, config, log

pytestmark = pytest.mark.gpu


def _rows(n, rng):
    base = {0, 1, 255, 256, 511, 512, 1023, n // 2, n - 1}
    base |= set(rng.choice(n, size=8, replace=False).tolist())
    return np.array(sorted(x for x in base if 0 <= x < n))


@pytest.mark.parametrize("shared", [True, False], ids=["shared_decode", "per_request_decode"])
def test_config5_pair_on_two_streams(shared):
    m = config(5)
    log(f"config 5 pair on two streams, shared decode={shared}")
    k, v = upload_pool(m.prefill.k_pool, m.prefill.v_pool)
    dd = prepare(m.decode, k, v, shared=shared)
    dp = prepare(m.prefill, k, v)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for _ in range(3):  # the bench's pattern, repeated: later launches overwrite earlier ones
        ev = torch.cuda.Event()
        ev.record(main)
        side.wait_event(ev)
        dd.run(side)
        dp.run(main)
        e2 = torch.cuda.Event()
        e2.record(side)
        main.wait_event(e2)
    torch.cuda.synchronize()
    od, ld = dd.out_f32(), dd.lse.cpu().numpy()
    op, lp = dp.out_f32(), dp.lse.cpu().numpy()
    reqs = list(range(0, 128, 11))
    rd = run_decode(m.decode, requests=reqs)
    for r in reqs:
        assert_parity(od[r], rd[r][0], "bf16", f"pair decode req {r}")
        assert_lse(ld[r], rd[r][1], "bf16", f"pair decode req {r}")
    rng = np.random.default_rng(55)
    rows = {r: _rows(m.prefill.q_len(r), rng) for r in range(m.prefill.batch)}
    rp = run_prefill(m.prefill, rows=rows)
    for r in range(m.prefill.batch):
        a = int(m.prefill.cu_q[r])
        assert_parity(op[a + rows[r]], rp[r][0], "bf16", f"pair prefill req {r}")
        assert_lse(lp[a + rows[r]], rp[r][1], "bf16", f"pair prefill req {r}")
