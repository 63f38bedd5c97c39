"""C-ABI host layer on the CPU: exports, cos/sin table, packing, validation, errors.

No kernel is launched here: every call either is host-only or fails argument
validation before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import position_agnostic_kv_lazy_amd as la
from position_agnostic_kv_lazy_amd import binding as B
from workloads import Segment, make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lazy_attn.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"LA_API\s+[\w\s\*]+?\b(lazy_attn_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 15, names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_status_strings():
    assert la.lazy_attn_status_string(0) == "LA_OK"
    assert la.lazy_attn_status_string(3) == "LA_ERR_WORKSPACE_TOO_SMALL"
    assert la.lazy_attn_status_string(99) == "LA_ERR_UNKNOWN"


def test_params_struct_layout():
    # int32 x4, int64, int32, float, int32 x5, int32[3] -> 64 bytes, int64 at offset 16
    assert ctypes.sizeof(B.la_params) == 64
    assert B.la_params.num_blocks.offset == 16


def test_rope_table_matches_oracle_definition():
    from oracle import rope_theta
    D, rows, base = 128, 70000, 5e5
    t = la.lazy_attn_rope_table(base, D, rows)
    th = rope_theta(D, base)
    for p in (0, 1, 15, 5184, 65535, 69999):
        ang = p * th
        np.testing.assert_allclose(t[p, :64], np.cos(ang), atol=6e-8, rtol=0)
        np.testing.assert_allclose(t[p, 64:], np.sin(ang), atol=6e-8, rtol=0)
    # float32 rounding of the float64 value: exact to half an ulp
    ref = np.cos(69999 * th).astype(np.float32)
    np.testing.assert_array_equal(t[69999, :64], ref)


def test_rope_table_errors():
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG"):
        la.lazy_attn_rope_table(1.0, 128, 10)
    with pytest.raises(la.LazyAttnError, match="even"):
        la.lazy_attn_rope_table(1e4, 127, 10)


def _params(**kw):
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=1000,
             dtype="bf16", scale=0.088, max_pos=20000)
    d.update(kw)
    return la.make_params(**d)


def _unpack(words):
    w = words.astype(np.uint64)
    return (w & np.uint64(0xFFFFFFFF)).astype(np.int64), \
        ((w >> np.uint64(32)) & np.uint64(0xFFFFFF)).astype(np.int64), \
        ((w >> np.uint64(56)) & np.uint64(0x7F)).astype(np.int64) + 1, \
        (w >> np.uint64(63)).astype(np.int64)


def test_pack_segments_round_trip():
    w = make_config(3, scale_down=4)
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    words, rbs, maxb = la.lazy_attn_pack_segments(p, w.requests)
    ids, pos0, nv, causal = _unpack(words)
    assert rbs[0] == 0 and len(rbs) == w.batch + 1
    assert maxb == int(np.max(np.diff(rbs)))
    for r, segs in enumerate(w.requests):
        row = rbs[r]
        for s in segs:
            for k, b in enumerate(s.blocks):
                assert ids[row] == b and pos0[row] == s.start + 16 * k
                assert nv[row] == min(16, s.n_tokens - 16 * k)
                assert causal[row] == int(s.is_new)
                row += 1
        assert row == rbs[r + 1]


def test_pack_segments_partial_blocks():
    p = _params(num_blocks=10, max_pos=100)
    segs = [[Segment(3, 20, np.array([4, 2]), False), Segment(60, 5, np.array([9]), True)]]
    words, rbs, _ = la.lazy_attn_pack_segments(p, segs)
    ids, pos0, nv, causal = _unpack(words)
    assert list(ids) == [4, 2, 9] and list(pos0) == [3, 19, 60]
    assert list(nv) == [16, 4, 5] and list(causal) == [0, 0, 1]


@pytest.mark.parametrize("segs,msg", [
    ([[Segment(0, 20, np.array([4]), False)]], "needs 2"),
    ([[Segment(0, 5, np.array([10]), False)]], "block id 10"),
    ([[Segment(98, 5, np.array([1]), False)]], "max_pos"),
    ([[Segment(-1, 5, np.array([1]), False)]], "outside"),
    ([[Segment(0, 0, np.array([], np.int64), False)]], "0 tokens"),
    ([[]], "no keys"),
])
def test_pack_segments_rejects(segs, msg):
    p = _params(num_blocks=10, max_pos=100)
    with pytest.raises(la.LazyAttnError, match=msg):
        la.lazy_attn_pack_segments(p, segs)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(num_kv_heads=5), "INVALID_ARG", "multiple"),
    (dict(head_dim=64), "UNSUPPORTED", "head_dim 128"),
    (dict(block_size=32), "UNSUPPORTED", "block_size 16"),
    (dict(num_q_heads=24), "UNSUPPORTED", "group sizes"),
    (dict(dtype=7), "UNSUPPORTED", "dtype"),
    (dict(max_pos=0), "INVALID_ARG", "max_pos"),
    (dict(num_blocks=0), "INVALID_ARG", "num_blocks"),
    (dict(scale=float("nan")), "INVALID_ARG", "scale"),
])
def test_param_validation(kw, status, msg):
    p = _params(**kw)
    with pytest.raises(la.LazyAttnError, match=f"{status}.*{msg}"):
        la.lazy_attn_decode_workspace_size(p, 4, 10)


@pytest.mark.parametrize("i", [0, 1])
def test_reserved_fields_must_be_zero(i):
    p = _params()
    p.reserved[i] = 1
    with pytest.raises(la.LazyAttnError, match="reserved"):
        la.lazy_attn_decode_workspace_size(p, 4, 10)
    p = _params()
    p.check_tables = 1  # the debugging switch is a field of its own
    assert la.lazy_attn_decode_workspace_size(p, 4, 10) >= 0


def test_fp32_mode_allows_head_dim_64():
    p = _params(dtype="f32", head_dim=64, num_q_heads=1, num_kv_heads=1)
    assert la.lazy_attn_decode_workspace_size(p, 1, 10) == 0


def test_workspace_size_formula():
    p = _params()
    # cfg2 shape: 64 requests x 8 kv heads = 512 pairs fill the default target of
    # 512 workgroups: one group per pair, no workspace, no combine
    assert la.lazy_attn_decode_workspace_size(p, 64, 324) == 0
    # fewer pairs: 32 x 8 = 256 pairs -> 2 groups each
    assert la.lazy_attn_decode_workspace_size(p, 32, 324) == 32 * 32 * 2 * 130 * 4
    # an explicit target
    p1 = _params(target_workgroups=1024)
    assert la.lazy_attn_decode_workspace_size(p1, 64, 324) == 64 * 32 * 2 * 130 * 4
    # explicit split size
    p2 = _params(split_blocks=100)
    assert la.lazy_attn_decode_workspace_size(p2, 64, 324) == 64 * 32 * 4 * 130 * 4
    # long context: 16 x 8 pairs, 4096 blocks -> 4 groups
    assert la.lazy_attn_decode_workspace_size(p, 16, 4096) == 16 * 32 * 4 * 130 * 4
    # short requests cap the split: at least 32 blocks per group (8 per wave)
    assert la.lazy_attn_decode_workspace_size(p, 1, 64) == 1 * 32 * 2 * 130 * 4


def test_validate_table_host_arrays():
    w = make_config(2, scale_down=8)
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    words, rbs, _ = la.lazy_attn_pack_segments(p, w.requests)
    qpos = w.q_pos.astype(np.int32)
    la.lazy_attn_validate_table(p, w.batch, words, rbs, qpos)
    bad = qpos.copy()
    bad[1] = w.table_rows()
    with pytest.raises(la.LazyAttnError, match="query positions"):
        la.lazy_attn_validate_table(p, w.batch, words, rbs, bad)
    p_small = _params(num_blocks=10, max_pos=w.table_rows())
    with pytest.raises(la.LazyAttnError, match="num_blocks"):
        la.lazy_attn_validate_table(p_small, w.batch, words, rbs, qpos)


def test_validate_table_reads_absolute_rows():
    """Rows are blk_words[b] for b in [req_blk_start[0], req_blk_start[batch]), the
    indices the kernels use, also when the first request does not start at row 0
    (a sub-batch slice of one CSR table)."""
    p = _params(num_blocks=10, max_pos=100)
    segs = [[Segment(0, 16, np.array([1]), False)],
            [Segment(0, 32, np.array([2, 3]), False)],
            [Segment(0, 16, np.array([4]), False)]]
    words, rbs, _ = la.lazy_attn_pack_segments(p, segs)
    qpos = np.array([40, 40, 40], np.int32)
    la.lazy_attn_validate_table(p, 3, words, rbs, qpos)
    # requests 1 and 2 alone, rows 1 .. 3 of the same table
    sub = rbs[1:].copy()
    la.lazy_attn_validate_table(p, 2, words, sub, qpos[1:])
    # a bad block id in the slice's last row must be caught ...
    bad = words.copy()
    bad[3] = (bad[3] & ~np.uint64(0xFFFFFFFF)) | np.uint64(12)
    with pytest.raises(la.LazyAttnError, match="block id 12"):
        la.lazy_attn_validate_table(p, 2, bad, sub, qpos[1:])
    # ... and so must a bad position there
    bad = words.copy()
    bad[3] = (bad[3] & ~(np.uint64(0xFFFFFF) << np.uint64(32))) | (np.uint64(95) << np.uint64(32))
    with pytest.raises(la.LazyAttnError, match="position 110"):
        la.lazy_attn_validate_table(p, 2, bad, sub, qpos[1:])


def test_validate_table_checks_launch_bounds():
    """Requests longer than the max_blocks_per_req / max_q_per_req a launch is sized
    from would be cut short silently: the validator rejects them."""
    p = _params(num_blocks=10, max_pos=200)
    segs = [[Segment(0, 16, np.array([1]), False)],
            [Segment(0, 40, np.array([2, 3, 4]), False)]]
    words, rbs, maxb = la.lazy_attn_pack_segments(p, segs)
    assert maxb == 3
    qpos = np.array([60, 60], np.int32)
    la.lazy_attn_validate_table(p, 2, words, rbs, qpos, None, 3)
    with pytest.raises(la.LazyAttnError, match="max_blocks_per_req 2"):
        la.lazy_attn_validate_table(p, 2, words, rbs, qpos, None, 2)
    with pytest.raises(la.LazyAttnError, match="must be >= 0"):
        la.lazy_attn_validate_table(p, 2, words, rbs, qpos, None, -1)
    cu = np.array([0, 5, 25], np.int32)
    la.lazy_attn_validate_table(p, 2, words, rbs, qpos, cu, 3, 20)
    with pytest.raises(la.LazyAttnError, match="max_q_per_req 19"):
        la.lazy_attn_validate_table(p, 2, words, rbs, qpos, cu, 3, 19)


def test_validate_table_prefill_needs_visible_key():
    p = _params(num_blocks=10, max_pos=100)
    segs = [[Segment(50, 5, np.array([1]), True)]]
    words, rbs, _ = la.lazy_attn_pack_segments(p, segs)
    cu = np.array([0, 3], np.int32)
    la.lazy_attn_validate_table(p, 1, words, rbs, np.array([50], np.int32), cu)
    with pytest.raises(la.LazyAttnError, match="sees no key"):
        la.lazy_attn_validate_table(p, 1, words, rbs, np.array([40], np.int32), cu)


def test_null_pointers_rejected_before_launch():
    p = _params()
    with pytest.raises(la.LazyAttnError, match="NULL"):
        la.lazy_attn_decode(p, None, None, None, None, None, None, None, 1, 1, None)
    with pytest.raises(la.LazyAttnError, match="NULL"):
        la.lazy_attn_prefill(p, None, None, None, None, None, None, None, None, 1, 1, None)


def test_noalloc_decode_rejects_shapes_beyond_its_scratch_before_launch():
    """The allocation-free decode holds its partials in a fixed array: a shape
    whose partials exceed it fails with a clear message, before any HIP call."""
    txt = open(HEADER).read()
    m = re.search(r"#define LA_DECODE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == B.LA_DECODE_NOALLOC_SCRATCH_BYTES
    p = _params(split_blocks=8)  # 64 x 8 pairs, 4096 blocks: 512 groups per pair
    need = la.lazy_attn_decode_workspace_size(p, 64, 4096)
    assert need > B.LA_DECODE_NOALLOC_SCRATCH_BYTES
    fake = 1 << 40  # never dereferenced: the size check fails first
    with pytest.raises(la.LazyAttnError, match="WORKSPACE_TOO_SMALL.*fixed scratch"):
        la.lazy_attn_decode_noalloc(p, fake, fake, fake, fake, fake, fake, fake, 64, 4096, fake)
    with pytest.raises(la.LazyAttnError, match="NULL"):
        la.lazy_attn_decode_noalloc(p, None, None, None, None, None, None, None, 1, 1, None)


def test_workspace_too_small_rejected_before_launch():
    p = _params()
    # 32 requests x 8 kv heads need 2 groups per pair, hence a workspace
    assert la.lazy_attn_decode_workspace_size(p, 32, 324) > 0
    fake = 1 << 40  # never dereferenced: the size check fails first
    with pytest.raises(la.LazyAttnError, match="WORKSPACE_TOO_SMALL"):
        la.lazy_attn_decode(p, fake, fake, fake, fake, fake, fake, fake, 32, 324, fake,
                            None, None, None)


def test_pack_segments_doc_local_words_carry_segment_start():
    p = _params(num_blocks=10, max_pos=100, pool_mode="doc_local")
    segs = [[Segment(3, 20, np.array([4, 2]), False), Segment(60, 5, np.array([9]), False)]]
    words, rbs, _ = la.lazy_attn_pack_segments(p, segs)
    ids, pos0, nv, _ = _unpack(words)
    assert list(ids) == [4, 2, 9] and list(pos0) == [3, 3, 60] and list(nv) == [16, 4, 5]
    la.lazy_attn_validate_table(p, 1, words, rbs, np.array([70], np.int32))


def test_pool_mode_checks():
    p = _params(pool_mode=2)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*pool_mode"):
        la.lazy_attn_decode_workspace_size(p, 4, 10)
    # doc-local: decode tables may not flag blocks causal; prefill causal
    # blocks must start blocks of the new-token segment at q_pos0
    p = _params(num_blocks=10, max_pos=100, pool_mode="doc_local")
    segs = [[Segment(3, 20, np.array([4, 2]), False), Segment(23, 20, np.array([5, 6]), True)]]
    words, rbs, _ = la.lazy_attn_pack_segments(p, segs)
    _, pos0, _, causal = _unpack(words)
    assert list(pos0) == [3, 3, 23, 39] and list(causal) == [0, 0, 1, 1]
    with pytest.raises(la.LazyAttnError, match="must not flag"):
        la.lazy_attn_validate_table(p, 1, words, rbs, np.array([50], np.int32))
    cu = np.array([0, 20], np.int32)
    la.lazy_attn_validate_table(p, 1, words, rbs, np.array([23], np.int32), cu)
    with pytest.raises(la.LazyAttnError, match="new-token segment"):
        la.lazy_attn_validate_table(p, 1, words, rbs, np.array([24], np.int32), cu)


def test_store_kv_argument_checks():
    p = _params()
    la.lazy_attn_store_kv(p, None, None, 0, None, None, None, None, None)  # empty: no-op
    with pytest.raises(la.LazyAttnError, match="n_tokens"):
        la.lazy_attn_store_kv(p, 1, 1, -1, 1, None, None, 1, 1)
    with pytest.raises(la.LazyAttnError, match="NULL"):
        la.lazy_attn_store_kv(p, None, 1, 4, 1, None, None, 1, 1)
    with pytest.raises(la.LazyAttnError, match="cos_sin"):
        la.lazy_attn_store_kv(p, 16, 16, 4, 16, 16, None, 16, 16)
    with pytest.raises(la.LazyAttnError, match="aligned"):
        la.lazy_attn_store_kv(p, 16, 18, 4, 16, None, None, 16, 16)


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch must not load a second HIP runtime."""
    import subprocess
    import sys
    code = ("import position_agnostic_kv_lazy_amd, torch\n"
            "print(sum(1 for l in open('/proc/self/maps') if 'libamdhip64' in l and 'r-xp' in l))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout.strip()
    assert out == "1", out


def test_alibi_slopes_match_oracle():
    from oracle import alibi_slopes
    for n in (1, 8, 12, 32, 71):
        got = la.lazy_attn_alibi_slopes(n)
        np.testing.assert_allclose(got, alibi_slopes(n), rtol=2e-7, atol=0)
    with pytest.raises(la.LazyAttnError, match="num_heads"):
        la.lazy_attn_alibi_slopes(0)


def test_pos_encoding_checks():
    with pytest.raises(la.LazyAttnError, match="pos_encoding"):
        la.lazy_attn_decode_workspace_size(_params(pos_encoding=3), 4, 10)
    with pytest.raises(la.LazyAttnError, match="ALiBi reads position-free"):
        la.lazy_attn_decode_workspace_size(_params(pos_encoding="alibi", pool_mode="doc_local"),
                                           4, 10)
    for enc in ("rope_half", "rope_interleaved", "alibi"):
        la.lazy_attn_decode_workspace_size(_params(pos_encoding=enc), 4, 10)


@pytest.mark.parametrize("sc", [
    {"type": "linear", "factor": 4.0},
    {"type": "ntk", "factor": 4.0},
    {"type": "yarn", "factor": 16.0, "original_max_pos": 4096, "beta_fast": 32.0, "beta_slow": 1.0},
    {"type": "yarn", "factor": 4.0, "original_max_pos": 8192, "beta_fast": 32.0, "beta_slow": 1.0,
     "attn_factor": 1.3},
    {"type": "yarn", "factor": 16.0, "original_max_pos": 65536, "beta_fast": 32.0,
     "beta_slow": 1.0},
    {"type": "llama3", "factor": 8.0, "original_max_pos": 8192, "low_freq_factor": 1.0,
     "high_freq_factor": 4.0},
], ids=lambda d: d["type"])
def test_scaled_table_matches_oracle(sc):
    from oracle import rope_theta_scaled
    D, rows, base = 128, 140000, 5e5
    t = la.lazy_attn_rope_table_scaled(base, D, rows, sc)
    th, amp = rope_theta_scaled(D, base, sc)
    for p in (0, 1, 4097, 65535, 139999):
        ang = p * th
        np.testing.assert_allclose(t[p, :64], amp * np.cos(ang), atol=1.5e-7, rtol=0)
        np.testing.assert_allclose(t[p, 64:], amp * np.sin(ang), atol=1.5e-7, rtol=0)


def test_scaled_table_none_is_plain_table():
    a = la.lazy_attn_rope_table(1e4, 64, 1000)
    b = la.lazy_attn_rope_table_scaled(1e4, 64, 1000, None)
    c = la.lazy_attn_rope_table_scaled(1e4, 64, 1000, {"type": "none"})
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
    with pytest.raises(la.LazyAttnError, match="factor"):
        la.lazy_attn_rope_table_scaled(1e4, 64, 10, {"type": "linear", "factor": 0.0})
    with pytest.raises(la.LazyAttnError, match="scaling type"):
        la.lazy_attn_rope_table_scaled(1e4, 64, 10, {"type": 9, "factor": 2.0})


def test_error_message_is_per_thread():
    import threading
    msgs = {}

    def fail(tag, fn):
        try:
            fn()
        except la.LazyAttnError:
            pass
        msgs[tag] = la.lazy_attn_last_error()

    t1 = threading.Thread(target=fail, args=("a", lambda: la.lazy_attn_alibi_slopes(0)))
    t1.start(); t1.join()
    t2 = threading.Thread(target=fail, args=("b", lambda: la.lazy_attn_rope_table(1.0, 64, 4)))
    t2.start(); t2.join()
    assert "num_heads" in msgs["a"] and "base" in msgs["b"]
    la.lazy_attn_alibi_slopes(4)
    assert la.lazy_attn_last_error() == ""  # success clears this thread's message
