"""The seeded input generators: shapes, determinism and NaN sentinel placement."""
import numpy as np
import pytest

import workloads


def _check_structure(wl):
    R, T = wl.num_reqs, wl.num_tokens
    nan_pool = np.isnan(wl.pool.astype(np.float32)) if wl.dtype == "f32" else \
        (wl.pool == workloads.BF16_NAN)
    poison = wl.num_blocks - 1
    assert nan_pool[:, poison].all()
    used = set()
    for r in range(R):
        L, c = int(wl.seq_lens[r]), int(wl.num_computed_tokens[r])
        nb = (L + 15) // 16
        row = wl.block_table[r]
        assert (row[nb:] == poison).all()
        blocks = row[:nb].tolist()
        assert not (set(blocks) & used)
        used |= set(blocks)
        for t in range(nb * 16):
            b, o = row[t // 16], t % 16
            if t < c:
                assert not nan_pool[:, b, o].any()          # cached context is live
            else:
                assert nan_pool[:, b, o].all()              # new-token slots and tail
    sm = wl.slot_mapping
    assert sm.shape == (T,) and len(set(sm.tolist())) == T
    for r in range(R):
        c = int(wl.num_computed_tokens[r])
        for i, t in enumerate(range(wl.query_start_loc[r], wl.query_start_loc[r + 1])):
            p = c + i
            assert sm[t] == wl.block_table[r, p // 16] * 16 + p % 16
    assert wl.q.shape == (T, wl.num_q_heads, wl.head_dim)
    assert wl.k_new.shape == wl.v_new.shape == (T, wl.num_kv_heads, wl.head_dim)


def test_tiny_workload_structure_and_determinism():
    a = workloads.build(workloads.BENCH_WORKLOADS[1])
    b = workloads.build(workloads.BENCH_WORKLOADS[1])
    assert a.dtype == "f32" and a.num_reqs == 4 and a.num_blocks == 65
    assert ((a.seq_lens >= 1) & (a.seq_lens <= 64)).all()
    _check_structure(a)
    for x, y in ((a.q, b.q), (a.pool, b.pool), (a.block_table, b.block_table)):
        assert x.tobytes() == y.tobytes()


@pytest.mark.parametrize("reqs", [[(0, 1)], [(0, 40), (16, 1), (5, 11)], [(31, 1), (32, 1), (0, 16)]])
def test_small_specs_structure(reqs):
    _check_structure(workloads.build(workloads.small_spec("s", 3, "bf16", 4, 2, 8, reqs)))


def test_workload_request_shapes():
    for n, spec in workloads.BENCH_WORKLOADS.items():
        reqs = spec.requests(np.random.default_rng([spec.seed, 0]))
        ql = np.array([q for _, q in reqs])
        L = np.array([c + q for c, q in reqs])
        if n == 2:
            assert len(reqs) == 64 and (ql == 1).all() and L.min() >= 512 and L.max() <= 4096
        if n == 3:
            assert len(reqs) == 256 and L.min() >= 16 and L.max() <= 8192
            assert 700 < np.median(L) < 1500
        if n == 4:
            assert ql.sum() == 8192 and len(reqs) == 2051
            assert [c for c, _ in reqs[:3]] == [0, 1024, 4096]
        if n == 5:
            assert (L == 32768).all() and len(reqs) == 8
