"""The seeded input generator: determinism, bf16 encoding and config sizes."""
import numpy as np
import pytest

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_config, zipf_probs


def test_bf16_round_trip_and_rounding():
    x = np.array([1.0, -2.5, 1.00390625, 1.005859375, 3.0e-3], np.float32)
    b = f32_to_bf16_bits(x)
    y = bf16_bits_to_f32(b)
    np.testing.assert_array_equal(f32_to_bf16_bits(y), b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to even (1.0)
    assert y[2] == 1.0
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    assert y[3] == np.float32(1.0078125)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)


def test_zipf_probs():
    p = zipf_probs(5, 1.0)
    assert p.sum() == pytest.approx(1.0)
    assert p[0] / p[1] == pytest.approx(2.0)


def test_config1_layout():
    w = make_config(1)
    assert w.dtype == "f32" and w.head_dim == 64 and w.num_blocks == 10
    assert [s.start for s in w.requests[0]] == [0, 32, 64, 96, 128]
    assert [list(s.blocks) for s in w.requests[0]][-1] == [8, 9]
    assert int(w.q_pos[0]) == 160


def test_config2_sizes_and_determinism():
    w = make_config(2)
    assert w.batch == 64 and w.num_blocks == 200 * 32 + 64 * 4
    assert set(w.keys_per_request()) == {5184}
    assert w.logical_kv_bytes() == 64 * 5184 * 4096
    w2 = make_config(2)
    np.testing.assert_array_equal(w.k_pool[:40], w2.k_pool[:40])
    np.testing.assert_array_equal(w.q, w2.q)
    for a, b in zip(w.requests[5], w2.requests[5]):
        assert a.start == b.start and list(a.blocks) == list(b.blocks)
    # documents are distinct within a request
    for segs in w.requests:
        docs = [int(s.blocks[0]) // 32 for s in segs[:-1]]
        assert len(set(docs)) == len(docs) == 10


def test_config3_flops():
    w = make_config(3)
    assert w.batch == 8 and w.q.shape == (8 * 512, 32, 128)
    expected = 8 * 32 * (4 * 512 * 10240 * 128 + 4 * (512 * 513 // 2) * 128)
    assert w.prefill_flops() == expected  # 704.4 GFLOP
    assert int(w.q_pos[0]) == 10240


def test_config5_shares_one_pool():
    m = make_config(5, scale_down=8)
    assert m.decode.k_pool is m.prefill.k_pool
    used = {int(b) for segs in m.decode.requests for s in segs for b in s.blocks}
    assert max(used) < m.prefill.meta["n_doc_blocks"]
