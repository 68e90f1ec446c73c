"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: hand-worked
fixtures, a scalar brute force over independently drawn contiguous K/V,
PyTorch's fp64 SDPA, closed forms and invariants that the definition implies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers: place contiguous per-request K/V into a scattered pool (test-side
# construction through the oracle's own write, then pinned separately).

def _scatter_requests(rng, Ks, Vs, ctxs, Hkv, D, dtype, extra_blocks=3):
    """Ks[r], Vs[r]: [L_r, Hkv, D] storage values. Returns pool, block_table."""
    nblk = [(len(K) + 15) // 16 for K in Ks]
    NB = sum(nblk) + extra_blocks
    perm = rng.permutation(NB)
    MB = max(nblk) + 1
    bt = np.full((len(Ks), MB), NB - 1, dtype=np.int32)
    store = np.uint16 if dtype == "bf16" else np.float32
    nan = workloads.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    pool = np.full((2, NB, 16, Hkv, D), nan, dtype=store)
    pos = 0
    for r, K in enumerate(Ks):
        bt[r, : nblk[r]] = perm[pos: pos + nblk[r]]
        pos += nblk[r]
        L = len(K)
        slots = np.array([bt[r, t // 16] * 16 + t % 16 for t in range(L)], dtype=np.int64)
        pool = oracle.kv_write(pool, K, Vs[r], slots)
    return pool, bt


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return workloads.bf16_bits_from_f32(x) if dtype == "bf16" else x


def _ragged_case(seed, dtype, Hq, Hkv, D, reqs):
    """reqs: list of (computed, qlen). Returns dict with contiguous and paged views."""
    rng = np.random.default_rng(seed)
    Ks = [_draw(rng, (c + ql, Hkv, D), dtype) for c, ql in reqs]
    Vs = [_draw(rng, (c + ql, Hkv, D), dtype) for c, ql in reqs]
    qs = [_draw(rng, (ql, Hq, D), dtype) for c, ql in reqs]
    pool, bt = _scatter_requests(rng, Ks, Vs, [c for c, _ in reqs], Hkv, D, dtype)
    qsl = np.zeros(len(reqs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([ql for _, ql in reqs])
    q = np.concatenate(qs) if qs else np.zeros((0, Hq, D), np.float32)
    return dict(Ks=Ks, Vs=Vs, qs=qs, q=q, pool=pool, bt=bt, qsl=qsl,
                nct=np.array([c for c, _ in reqs], np.int32),
                L=np.array([c + ql for c, ql in reqs], np.int32))


def _run(case, scale, dtype):
    return oracle.attention(case["q"], case["pool"], case["bt"], case["L"], case["qsl"],
                            case["nct"], scale, dtype)


# ---------------------------------------------------------------------------
# storage formats

def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_generator_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 7.0
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties to even
    ours = workloads.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_round_to_storage_bf16_hand_worked():
    """float32 bit patterns -> bf16 bits, each worked out by hand from the
    rule (keep the top 16 bits; round the low 16 to nearest, ties to even)."""
    cases = [
        (0x3F800000, 0x3F80),   # 1.0 exactly
        (0x3F808000, 0x3F80),   # 1 + 2^-8: a tie, kept mantissa even -> down
        (0x3F818000, 0x3F82),   # 1 + 3*2^-8: a tie, kept mantissa odd -> up
        (0x3F808001, 0x3F81),   # just above the tie -> up
        (0x3F807FFF, 0x3F80),   # just below the tie -> down
        (0xBF818000, 0xBF82),   # sign does not change the magnitude rule
        (0x3FFFFFFF, 0x4000),   # 1.99999988: mantissa carry bumps the exponent -> 2.0
        (0x7F7FFFFF, 0x7F80),   # largest finite float32 rounds up to +inf
        (0x7F7F7FFF, 0x7F7F),   # below the tie stays the largest finite bf16
        (0x00008000, 0x0000),   # subnormal tie, even -> +0
        (0x00018000, 0x0002),   # subnormal tie, odd -> up
        (0x80008000, 0x8000),   # negative subnormal tie -> -0
        (0x007FFFFF, 0x0080),   # largest subnormal carries into the smallest normal
        (0x7F800000, 0x7F80),   # +inf
        (0xFF800000, 0xFF80),   # -inf
    ]
    f32 = np.array([c for c, _ in cases], np.uint32).view(np.float32)
    got = oracle.round_to_storage(f32.astype(np.float64), "bf16")
    assert got.tolist() == [b for _, b in cases]
    # NaN stays NaN, whatever its payload (a plain add-and-shift would turn
    # 0x7F800001 into infinity and wrap 0xFFFFFFFF round to zero)
    nans = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0xFF800001], np.uint32).view(np.float32)
    got = oracle.round_to_storage(nans.astype(np.float64), "bf16")
    assert np.isnan(oracle.bf16_bits_to_f64(got)).all()


def test_round_to_storage_goes_through_float32():
    # 1 + 2^-8 + 2^-40 rounds to float32 1 + 2^-8, a bf16 tie, which goes down
    # to 1.0 (rounding the float64 straight to bf16 would give 1 + 2^-7)
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24])
    assert oracle.round_to_storage(x[:1], "bf16").tolist() == [0x3F80]
    f = oracle.round_to_storage(x[1:], "f32")
    assert f.dtype == np.float32
    assert f.tolist() == [1.0, 1 + 2.0 ** -22]       # float32 ties to even


def test_round_to_storage_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, 400000, dtype=np.uint64).astype(np.uint32)
    bits[:65536] = (np.arange(65536, dtype=np.uint32) << 16) | 0x8000     # every tie
    f32 = bits.view(np.float32)
    x = np.concatenate([f32.astype(np.float64), rng.standard_normal(100000) * 1e3,
                        rng.standard_normal(1000) * 1e39])               # beyond float32: +-inf
    ours = oracle.round_to_storage(x, "bf16")
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert (ours[~nan] == ref[~nan]).all()
    assert (ours[nan] == 0x7FC0).all()
    ref32 = torch.from_numpy(x).to(torch.float32).numpy()
    f = oracle.round_to_storage(x, "f32")
    assert (f.view(np.uint32)[~nan] == ref32.view(np.uint32)[~nan]).all()


# ---------------------------------------------------------------------------
# golden fixtures (hand-worked)

def test_golden_slot_arithmetic():
    g = json.load(open(os.path.join(GOLDEN, "slot_arithmetic.json")))
    fo = g["flat_offsets"]
    NB, Hkv, D = fo["num_blocks"], fo["num_kv_heads"], fo["head_dim"]
    for c in g["slots"]:
        pool = np.zeros((2, NB, 16, 1, 1), np.float32)
        k = np.array([[[1.0]]], np.float32)
        v = np.array([[[2.0]]], np.float32)
        out = oracle.kv_write(pool, k, v, np.array([c["slot"]], np.int64))
        assert out[0, c["block"], c["offset"], 0, 0] == 1.0
        assert out[1, c["block"], c["offset"], 0, 0] == 2.0
        assert np.count_nonzero(out) == 2
    for c in fo["cases"]:
        pool = np.zeros((2, NB, 16, Hkv, D), np.float32)
        k = np.zeros((1, Hkv, D), np.float32)
        v = np.zeros((1, Hkv, D), np.float32)
        (k if c["kv"] == 0 else v)[0, c["head"], c["d"]] = 5.0
        out = oracle.kv_write(pool, k, v, np.array([c["slot"]], np.int64))
        assert np.flatnonzero(out.reshape(-1)).tolist() == [c["flat"]]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "closed_forms.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    q = np.array(case["q"], np.float64)
    K = np.array(case["k"], np.float64)
    V = np.array(case["v"], np.float64)
    ql, Hq, D = q.shape
    L, Hkv, _ = K.shape
    # place the L tokens in scattered blocks 3, 0 (block table [3, 0]) of a 4-block pool
    pool = np.full((2, 4, 16, Hkv, D), np.nan)
    bt = np.array([[3, 0]], np.int32)
    slots = np.array([bt[0, t // 16] * 16 + t % 16 for t in range(L)], np.int64)
    pool = oracle.kv_write(pool, K, V, slots)
    out = oracle.attention(q.astype(np.float32), pool.astype(np.float32), bt,
                           np.array([L], np.int32), np.array([0, ql], np.int32),
                           np.array([case["computed"]], np.int32), case["scale"], "f32")
    # inputs are float32-rounded, so compare at float32 input precision
    np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=2e-6)
    # exact fp64 check through the scalar brute force on the same values
    bf = oracle.dense_brute_force(q.tolist(), K.tolist(), V.tolist(), case["scale"], case["computed"])
    np.testing.assert_allclose(np.array(bf), np.array(case["out"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P1: dense brute force and torch SDPA

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (3, 3), (4, 1)])
def test_matches_scalar_brute_force(dtype, Hq, Hkv):
    reqs = [(0, 1), (5, 1), (17, 3), (0, 20), (31, 2)]
    case = _ragged_case(11, dtype, Hq, Hkv, 8, reqs)
    scale = 0.37
    out = _run(case, scale, dtype)
    for r, (c, ql) in enumerate(reqs):
        q = oracle.to_f64(case["qs"][r], dtype).tolist()
        K = oracle.to_f64(case["Ks"][r], dtype).tolist()
        V = oracle.to_f64(case["Vs"][r], dtype).tolist()
        bf = np.array(oracle.dense_brute_force(q, K, V, scale, c))
        np.testing.assert_allclose(out[case["qsl"][r]: case["qsl"][r + 1]], bf, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_fp64():
    reqs = [(7, 1), (0, 33), (40, 9), (100, 1)]
    Hq, Hkv, D = 8, 2, 16
    case = _ragged_case(5, "f32", Hq, Hkv, D, reqs)
    scale = 1 / math.sqrt(D)
    out = _run(case, scale, "f32")
    for r, (c, ql) in enumerate(reqs):
        q = torch.from_numpy(case["qs"][r].astype(np.float64)).permute(1, 0, 2)     # [Hq, ql, D]
        K = torch.from_numpy(case["Ks"][r].astype(np.float64)).permute(1, 0, 2)     # [Hkv, L, D]
        V = torch.from_numpy(case["Vs"][r].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        V = V.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        L = c + ql
        mask = torch.arange(L)[None, :] <= (c + torch.arange(ql))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[case["qsl"][r]: case["qsl"][r + 1]],
                                   ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P2: physical block permutation invariance

def test_block_permutation_invariance():
    wl = workloads.build(workloads.small_spec("perm", 3, "bf16", 4, 2, 16,
                                               [(40, 1), (0, 25), (70, 3)]))
    pool = oracle.kv_write(wl.pool, wl.k_new, wl.v_new, wl.slot_mapping)
    out = oracle.attention(wl.q, pool, wl.block_table, wl.seq_lens, wl.query_start_loc,
                           wl.num_computed_tokens, wl.scale, "bf16")
    NB = pool.shape[1]
    perm = np.random.default_rng(9).permutation(NB)
    pool2 = np.empty_like(pool)
    pool2[:, perm] = pool
    bt2 = perm[wl.block_table].astype(np.int32)
    out2 = oracle.attention(wl.q, pool2, bt2, wl.seq_lens, wl.query_start_loc,
                            wl.num_computed_tokens, wl.scale, "bf16")
    assert np.array_equal(out, out2)


# ---------------------------------------------------------------------------
# P3: softmax rows sum to one; V == 1 gives 1

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 4, 8))
    K = rng.standard_normal((30, 2, 8)) * 3
    w = oracle.request_weights(q, K, 24, 0.9, 4)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-12)
    # row i sees exactly 24 + i + 1 keys
    for i in range(6):
        assert np.all(w[i, :, 24 + i + 1:] == 0) and np.all(w[i, :, : 24 + i + 1] > 0)


def test_constant_v_gives_constant_out():
    case = _ragged_case(4, "f32", 4, 2, 8, [(9, 1), (0, 12)])
    pool = case["pool"].copy()
    finite = np.isfinite(pool[1])
    pool[1][finite] = 1.0
    case["pool"] = pool
    out = _run(case, 0.5, "f32")
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# P4, P5: single-token context returns V; zero query averages visible V

def test_single_token_context_returns_v():
    case = _ragged_case(6, "bf16", 4, 2, 8, [(0, 1), (0, 1)])
    out = _run(case, 0.125, "bf16")
    for r in range(2):
        v0 = oracle.to_f64(case["Vs"][r][0], "bf16")          # [Hkv, D]
        assert np.array_equal(out[r], v0[np.arange(4) // 2])


def test_zero_query_is_mean_of_visible_v():
    reqs = [(10, 4), (3, 1)]
    case = _ragged_case(7, "f32", 4, 2, 8, reqs)
    case["q"] = np.zeros_like(case["q"])
    out = _run(case, 1.0, "f32")
    for r, (c, ql) in enumerate(reqs):
        V = case["Vs"][r].astype(np.float64)
        for i in range(ql):
            mean = V[: c + i + 1].mean(axis=0)                  # [Hkv, D]
            np.testing.assert_allclose(out[case["qsl"][r] + i], mean[np.arange(4) // 2],
                                       rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# P6, P7: decode == last prefill row; chunk-split invariance

def test_decode_equals_last_prefill_row_and_chunk_invariance():
    rng = np.random.default_rng(8)
    Hq, Hkv, D, n = 4, 2, 8, 37
    K = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((n, Hq, D)).astype(np.float32)
    pool, bt = _scatter_requests(rng, [K], [V], [0], Hkv, D, "f32")
    L = np.array([n], np.int32)

    def run(c, ql):
        return oracle.attention(q[c: c + ql], pool, bt, np.array([c + ql], np.int32),
                                np.array([0, ql], np.int32), np.array([c], np.int32), 0.3, "f32")

    full = run(0, n)                       # one prefill of all n tokens
    dec = run(n - 1, 1)                    # decode of the last token
    np.testing.assert_allclose(dec[0], full[-1], rtol=0, atol=1e-13)
    for k in (1, 16, 20, 36):              # split into [0,k) and [k,n)
        a = run(0, k)
        b = run(k, n - k)
        np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=0, atol=1e-13)
    del L


# ---------------------------------------------------------------------------
# P8: split-KV merge equals the direct softmax

@pytest.mark.parametrize("partition", [1, 5, 16, 512, 10000])
def test_split_kv_merge(partition):
    rng = np.random.default_rng(partition)
    n, D = 1500, 16
    K = rng.standard_normal((n, D)) * 2
    V = rng.standard_normal((n, D))
    q = rng.standard_normal(D)
    s = K @ q * 0.25
    w = np.exp(s - s.max())
    direct = (w / w.sum()) @ V
    got = oracle.split_kv_row(q, K, V, 0.25, partition)
    np.testing.assert_allclose(got, direct, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P9: write round trip, sentinels untouched

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_round_trip(dtype):
    wl = workloads.build(workloads.small_spec("rt", 12, dtype, 4, 2, 16,
                                               [(0, 20), (33, 1), (5, 7), (15, 2)]))
    pool = oracle.kv_write(wl.pool, wl.k_new, wl.v_new, wl.slot_mapping)
    touched = np.zeros(pool.shape[1:3], bool)
    for t, s in enumerate(wl.slot_mapping):
        b, o = divmod(int(s), 16)
        touched[b, o] = True
        assert pool[0, b, o].tobytes() == wl.k_new[t].tobytes()
        assert pool[1, b, o].tobytes() == wl.v_new[t].tobytes()
    assert pool[:, ~touched].tobytes() == wl.pool[:, ~touched].tobytes()
    # -1 padding tokens are skipped
    sm = wl.slot_mapping.copy()
    sm[::2] = -1
    p2 = oracle.kv_write(wl.pool, wl.k_new, wl.v_new, sm)
    for t in range(0, len(sm), 2):
        b, o = divmod(int(wl.slot_mapping[t]), 16)
        assert p2[:, b, o].tobytes() == wl.pool[:, b, o].tobytes()


def test_write_rejects_out_of_pool_slot():
    pool = np.zeros((2, 2, 16, 1, 1), np.float32)
    kv = np.zeros((1, 1, 1), np.float32)
    for bad in (32, -2):
        with pytest.raises(ValueError):
            oracle.kv_write(pool, kv, kv, np.array([bad], np.int64))


# ---------------------------------------------------------------------------
# P10: MHA and MQA reduce to textbook per-head attention

@pytest.mark.parametrize("Hkv", [4, 1])
def test_mha_and_mqa(Hkv):
    Hq, D, c, ql = 4, 8, 6, 3
    case = _ragged_case(13, "f32", Hq, Hkv, D, [(c, ql)])
    out = _run(case, 0.5, "f32")
    K = case["Ks"][0].astype(np.float64)
    V = case["Vs"][0].astype(np.float64)
    q = case["qs"][0].astype(np.float64)
    for h in range(Hq):
        g = h if Hkv == Hq else 0
        S = q[:, h] @ K[:, g].T * 0.5                                    # [ql, L]
        S = S + np.where(np.arange(c + ql)[None] <= (c + np.arange(ql))[:, None], 0, -np.inf)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        np.testing.assert_allclose(out[:, h], P @ V[:, g], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# P11: request order invariance; empty requests

def test_request_order_invariance_and_empty_requests():
    reqs = [(3, 2), (0, 1), (20, 5), (8, 0), (47, 1)]
    case = _ragged_case(14, "f32", 4, 2, 8, reqs)
    out = _run(case, 0.4, "f32")
    order = [4, 3, 0, 2, 1]
    qs = [case["qs"][r] for r in order]
    qsl = np.zeros(len(order) + 1, np.int32)
    qsl[1:] = np.cumsum([reqs[r][1] for r in order])
    out2 = oracle.attention(np.concatenate(qs), case["pool"], case["bt"][order],
                            case["L"][order], qsl, case["nct"][order], 0.4, "f32")
    for j, r in enumerate(order):
        assert np.array_equal(out2[qsl[j]: qsl[j + 1]],
                              out[case["qsl"][r]: case["qsl"][r + 1]])


def test_rejects_inconsistent_metadata():
    case = _ragged_case(15, "f32", 2, 1, 4, [(3, 2)])
    with pytest.raises(ValueError):
        oracle.attention(case["q"], case["pool"], case["bt"], case["L"] + 1, case["qsl"],
                         case["nct"], 1.0, "f32")


def test_rows_agree_with_full():
    wl = workloads.build(workloads.small_spec("rows", 16, "bf16", 8, 2, 16,
                                               [(30, 1), (0, 18), (50, 6)]))
    pool = oracle.kv_write(wl.pool, wl.k_new, wl.v_new, wl.slot_mapping)
    args = (wl.q, pool, wl.block_table, wl.seq_lens, wl.query_start_loc,
            wl.num_computed_tokens, wl.scale, "bf16")
    full = oracle.attention(*args)
    rows = [0, 1, 5, 18, 19, 24]
    np.testing.assert_allclose(oracle.attention_rows(*args, tokens=rows), full[rows],
                               rtol=0, atol=1e-13)
    # runs of consecutive rows, across request boundaries, with every run length
    rows = list(range(wl.num_tokens))
    for run in (1, 2, 3, 5, 256):
        np.testing.assert_allclose(oracle.attention_rows(*args, tokens=rows, max_run=run), full,
                                   rtol=0, atol=1e-13)
    rows = [3, 4, 5, 6, 17, 18, 19, 20, 21, 22, 23, 24]
    np.testing.assert_allclose(oracle.attention_rows(*args, tokens=rows, max_run=3), full[rows],
                               rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Planted mistakes in a copy of the oracle are caught by the pins above.

def test_planted_mistakes_are_caught(monkeypatch):
    reqs = [(5, 1), (0, 6)]
    case = _ragged_case(17, "f32", 4, 2, 8, reqs)

    def brute(r):
        return np.array(oracle.dense_brute_force(
            case["qs"][r].astype(np.float64).tolist(), case["Ks"][r].astype(np.float64).tolist(),
            case["Vs"][r].astype(np.float64).tolist(), 0.5, reqs[r][0]))

    good = _run(case, 0.5, "f32")
    np.testing.assert_allclose(good[1:7], brute(1), atol=1e-12)

    # (a) GQA mapping by modulo instead of by group
    orig = oracle.request_weights

    def wrong_gqa(q_rows, K, computed, scale, num_q_heads):
        return orig(q_rows, K[:, ::-1], computed, scale, num_q_heads)
    monkeypatch.setattr(oracle, "request_weights", wrong_gqa)
    bad = _run(case, 0.5, "f32")
    assert not np.allclose(bad[1:7], brute(1), atol=1e-6)
    monkeypatch.undo()

    # (b) causal window off by one
    def wrong_mask(q_rows, K, computed, scale, num_q_heads):
        return orig(q_rows, K, computed - 1, scale, num_q_heads)
    monkeypatch.setattr(oracle, "request_weights", wrong_mask)
    with np.errstate(invalid="ignore"):
        bad = _run(case, 0.5, "f32")
    assert not np.allclose(bad[1:7], brute(1), atol=1e-6, equal_nan=False)
    monkeypatch.undo()

    # (c) block offset taken from the wrong end of the slot
    orig_gather = oracle.gather_kv

    def wrong_gather(pool, row, L, dtype, block_size=16):
        K, V = orig_gather(pool, row, L, dtype, block_size)
        return K, V[::-1].copy()
    monkeypatch.setattr(oracle, "gather_kv", wrong_gather)
    bad = _run(case, 0.5, "f32")
    assert not np.allclose(bad[1:7], brute(1), atol=1e-6)


# ---------------------------------------------------------------------------
# copy_blocks (copy-on-write): pointing a request's table at a copy of one of
# its blocks leaves what the request reads unchanged; nothing else changes.

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_blocks_preserves_logical_content(dtype):
    rng = np.random.default_rng(21)
    case = _ragged_case(21, dtype, 4, 2, 16, [(37, 1), (20, 5)])
    pool, bt = case["pool"], case["bt"].copy()
    NB = pool.shape[1]
    used = set(int(b) for r in range(2) for b in bt[r, : (int(case["L"][r]) + 15) // 16])
    spare = [b for b in range(NB) if b not in used][:2]
    pairs = [(int(bt[0, 1]), spare[0]), (int(bt[1, 0]), spare[1])]
    pool2 = oracle.copy_blocks(pool, pairs)
    bt2 = bt.copy()
    bt2[0, 1], bt2[1, 0] = spare
    for r in range(2):
        K1, V1 = oracle.gather_kv(pool, bt[r], int(case["L"][r]), dtype)
        K2, V2 = oracle.gather_kv(pool2, bt2[r], int(case["L"][r]), dtype)
        assert np.array_equal(K1, K2, equal_nan=True) and np.array_equal(V1, V2, equal_nan=True)
    untouched = [b for b in range(NB) if b not in spare]
    assert pool2[:, untouched].tobytes() == pool[:, untouched].tobytes()
    out1 = _run(case, 0.3, dtype)
    case2 = dict(case, pool=pool2, bt=bt2)
    assert np.array_equal(out1, _run(case2, 0.3, dtype))


# ---------------------------------------------------------------------------
# RoPE: hand-worked cases, the complex-number form, relative positions.

def _rope_cache(max_pos, rotary_dim, base=10000.0):
    inv = base ** (-np.arange(0, rotary_dim, 2, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def test_golden_rope():
    g = json.load(open(os.path.join(GOLDEN, "rope_cases.json")))
    cache = np.array([g["cos_sin_row"]], dtype=np.float32)
    for c in g["cases"]:
        x = np.array([[c["x"]]], dtype=np.float32)
        got = oracle.rope(x, np.array([0]), cache, g["rotary_dim"], c["is_neox"], "f32")[0, 0]
        assert np.allclose(got, c["expect"], atol=1e-6), (c, got)


@pytest.mark.parametrize("is_neox", [True, False])
def test_rope_matches_complex_rotation_and_keeps_norms(is_neox):
    rng = np.random.default_rng(5)
    T, H, D, r = 7, 3, 16, 12
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    pos = rng.integers(0, 50, T)
    cache = _rope_cache(64, r)
    got = oracle.rope(x, pos, cache, r, is_neox, "f32")
    half = r // 2
    ix = np.arange(half) if is_neox else 2 * np.arange(half)
    iy = ix + half if is_neox else ix + 1
    z = x[:, :, ix].astype(np.float64) + 1j * x[:, :, iy].astype(np.float64)
    e = cache[pos, :half].astype(np.float64) + 1j * cache[pos, half:r].astype(np.float64)
    zr = z * e[:, None, :]
    assert np.allclose(got[:, :, ix], zr.real, atol=1e-12) and np.allclose(got[:, :, iy], zr.imag, atol=1e-12)
    assert np.array_equal(got[:, :, r:], x[:, :, r:].astype(np.float64))
    assert np.allclose(np.abs(zr), np.abs(z) * np.abs(e[:, None, :]), atol=1e-12)


@pytest.mark.parametrize("is_neox", [True, False])
def test_rope_scores_depend_on_relative_position_only(is_neox):
    rng = np.random.default_rng(6)
    D = r = 32
    cache = _rope_cache(256, r)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)
    dots = []
    for m, n in [(10, 3), (40, 33), (200, 193)]:
        qm = oracle.rope(q, np.array([m]), cache, r, is_neox, "f32")
        kn = oracle.rope(k, np.array([n]), cache, r, is_neox, "f32")
        dots.append(float((qm * kn).sum()))
    assert max(dots) - min(dots) < 1e-4 * max(1.0, abs(dots[0]))
    # a different offset changes the score
    q0 = oracle.rope(q, np.array([10]), cache, r, is_neox, "f32")
    k0 = oracle.rope(k, np.array([2]), cache, r, is_neox, "f32")
    assert abs(float((q0 * k0).sum()) - dots[0]) > 1e-3


# ---------------------------------------------------------------------------
# INT8 KV cache: hand-worked codes, the error bound of the rounding, and
# attention over exactly representable values equals the unquantised oracle.

def test_golden_int8_quantisation():
    g = json.load(open(os.path.join(GOLDEN, "int8_quant.json")))
    x = np.array([r["x"] for r in g["rows"]], np.float32)
    codes, scales = oracle.quantize_int8(x, "f32")
    assert codes.tolist() == [r["codes"] for r in g["rows"]]
    assert scales.tolist() == [r["scale"] for r in g["rows"]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_int8_rounding_error_bound(dtype):
    rng = np.random.default_rng(8)
    x = _draw(rng, (50, 4, 128), dtype)
    codes, scales = oracle.quantize_int8(x, dtype)
    xf = oracle.to_f64(x, dtype)
    err = np.abs(oracle.dequantize_int8(codes, scales) - xf)
    # half a step, plus float32 rounding of the quotient
    assert np.all(err <= scales[..., None] * (0.5 + 1e-5) + 1e-30)
    amax_idx = np.abs(xf).argmax(axis=-1)
    assert np.all(np.abs(np.take_along_axis(codes, amax_idx[..., None], -1)) == 127)
    assert codes.min() >= -127


def test_int8_attention_equals_plain_on_representable_values():
    # values k * 2^-4 with |k| <= 127 and every row's max exactly 127 * 2^-4:
    # quantisation is then exact and INT8 attention must equal the plain one
    rng = np.random.default_rng(9)
    Hq, Hkv, D = 8, 2, 64
    reqs = [(30, 1), (0, 20), (60, 5)]
    def rep(shape):
        v = rng.integers(-126, 127, shape).astype(np.float32)
        v[..., 0] = 127.0
        return (v / 16).astype(np.float32)
    Ks = [rep((c + ql, Hkv, D)) for c, ql in reqs]
    Vs = [rep((c + ql, Hkv, D)) for c, ql in reqs]
    case = _ragged_case(9, "f32", Hq, Hkv, D, reqs)
    pool, bt = _scatter_requests(rng, Ks, Vs, [c for c, _ in reqs], Hkv, D, "f32")
    case = dict(case, Ks=Ks, Vs=Vs, pool=pool, bt=bt)
    NB = pool.shape[1]
    codes = np.zeros((2, NB, 16, Hkv, D), np.int8)
    scales = np.zeros((2, NB, 16, Hkv), np.float32)
    for r, (K, V) in enumerate(zip(Ks, Vs)):
        slots = np.array([bt[r, t // 16] * 16 + t % 16 for t in range(len(K))], np.int64)
        codes, scales = oracle.kv_write_int8(codes, scales, K, V, slots, "f32")
    ref = _run(case, 0.2, "f32")
    got = oracle.attention_int8(case["q"], codes, scales, bt, case["L"], case["qsl"], case["nct"], 0.2, "f32")
    assert np.allclose(got, ref, atol=1e-12, rtol=0)
    assert np.all(scales[:, bt[0, 0]][:, 0] == np.float32(1 / 16))   # max 127/16 over 127


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache: hand-worked decodes and codes from the format's
# definition, an independent round-to-nearest-even on the float32 bits, the
# error bound of the rounding, and attention over exactly representable values
# equals the unquantised oracle.

def test_golden_fp8_e4m3():
    g = json.load(open(os.path.join(GOLDEN, "fp8_e4m3.json")))
    for code, val in g["decode"]:
        got = float(oracle.fp8_e4m3_decode(np.array([int(code, 16)], np.uint8))[0])
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    x = np.array([r["x"] for r in g["rows"]], np.float32)
    codes, scales = oracle.quantize_fp8(x, "f32")
    assert codes.tolist() == [[int(c, 16) for c in r["codes"]] for r in g["rows"]]
    assert scales.tolist() == [r["scale"] for r in g["rows"]]


def _e4m3_rne_bits(y):
    """Round-to-nearest-even of float32 y (|y| <= 448) to E4M3 by integer
    arithmetic on the float32 bits: a second construction of the encoding."""
    out = []
    for v in np.asarray(y, np.float32).ravel():
        b = int(np.float32(v).view(np.uint32))
        sign = (b >> 24) & 0x80
        a = abs(float(v))
        if a < 2.0 ** -6:
            q = a * 512.0                       # subnormal steps of 2^-9
            n = int(np.floor(q))
            frac = q - n
            n += 1 if (frac > 0.5 or (frac == 0.5 and n % 2 == 1)) else 0
            code = n
        else:
            ab = b & 0x7FFFFFFF
            e = (ab >> 23) - 127 + 7
            mant = ab & 0x7FFFFF
            r, rem = mant >> 20, mant & 0xFFFFF
            r += 1 if (rem > 0x80000 or (rem == 0x80000 and r & 1)) else 0
            code = (e << 3) + r
        out.append(sign | code)
    return np.array(out, np.uint8).reshape(np.shape(y))


def test_fp8_encode_matches_bitwise_rne():
    rng = np.random.default_rng(11)
    mags = oracle.fp8_e4m3_magnitudes()
    ties = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)          # every midpoint (exact in float32)
    rand = (rng.standard_normal(4000) * rng.choice([1e-3, 0.05, 1, 30, 200], 4000)).astype(np.float32)
    rand = np.clip(rand, -448, 448).astype(np.float32)
    y = np.concatenate([ties, -ties, mags.astype(np.float32), rand, np.array([0.0, -0.0, 448.0], np.float32)])
    assert np.array_equal(oracle.fp8_e4m3_encode(y), _e4m3_rne_bits(y))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_rounding_error_bound(dtype):
    rng = np.random.default_rng(12)
    x = _draw(rng, (50, 4, 128), dtype)
    codes, scales = oracle.quantize_fp8(x, dtype)
    xf = oracle.to_f64(x, dtype)
    y = np.abs(xf) / np.where(scales > 0, scales, 1)[..., None]
    # half a step: 2^-4 relative for normals (3 mantissa bits), 2^-10 absolute below 2^-6
    step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 3), 2.0 ** -9)
    err = np.abs(oracle.dequantize_fp8(codes, scales) - xf)
    assert np.all(err <= scales[..., None] * (step / 2 * (1 + 1e-5) + 1e-6) + 1e-30)
    amax_idx = np.abs(xf).argmax(axis=-1)
    assert np.all(np.take_along_axis(codes, amax_idx[..., None], -1) & 0x7F == 0x7E)
    assert not np.any((codes & 0x7F) == 0x7F)


def test_fp8_attention_equals_plain_on_representable_values():
    # values (E4M3 value) * 2^-4 with every row's max exactly 448 * 2^-4:
    # quantisation is then exact and FP8 attention must equal the plain one
    rng = np.random.default_rng(13)
    Hq, Hkv, D = 8, 2, 64
    reqs = [(30, 1), (0, 20), (60, 5)]
    mags = oracle.fp8_e4m3_magnitudes()
    def rep(shape):
        v = mags[rng.integers(0, 126, shape)] * rng.choice([-1.0, 1.0], shape)
        v[..., 0] = 448.0
        return (v / 16).astype(np.float32)
    Ks = [rep((c + ql, Hkv, D)) for c, ql in reqs]
    Vs = [rep((c + ql, Hkv, D)) for c, ql in reqs]
    case = _ragged_case(13, "f32", Hq, Hkv, D, reqs)
    pool, bt = _scatter_requests(rng, Ks, Vs, [c for c, _ in reqs], Hkv, D, "f32")
    case = dict(case, Ks=Ks, Vs=Vs, pool=pool, bt=bt)
    NB = pool.shape[1]
    codes = np.zeros((2, NB, 16, Hkv, D), np.uint8)
    scales = np.zeros((2, NB, 16, Hkv), np.float32)
    for r, (K, V) in enumerate(zip(Ks, Vs)):
        slots = np.array([bt[r, t // 16] * 16 + t % 16 for t in range(len(K))], np.int64)
        codes, scales = oracle.kv_write_fp8(codes, scales, K, V, slots, "f32")
    ref = _run(case, 0.2, "f32")
    got = oracle.attention_fp8(case["q"], codes, scales, bt, case["L"], case["qsl"], case["nct"], 0.2, "f32")
    assert np.allclose(got, ref, atol=1e-12, rtol=0)
    assert np.all(scales[:, bt[0, 0]][:, 0] == np.float32(1 / 16))
