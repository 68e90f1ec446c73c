"""INT8 KV cache on the GPU against the fp64 oracle.

* paged_kv_write_int8: codes and scales bit for bit (both sides take the
  rounding decisions in IEEE float32), untouched slots unchanged.
* paged_attention_int8: decode rows, prefill rows and split-KV rows over
  the dequantised cache within the output tolerance, for bf16 and fp32 q,
  head_dim 64 / 128 and several GQA groups; unused slots hold garbage codes
  and NaN scales, which must never reach the output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_close, from_dev, out_f64, scales_from_dev, scales_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _quantised_pool(wl):
    """The workload's cache quantised row by row; NaN (unused) slots get
    garbage codes and NaN scales."""
    with np.errstate(invalid="ignore"):
        f = oracle.to_f64(wl.pool, wl.dtype)
    bad = np.isnan(f).any(axis=-1)
    clean = np.where(np.isnan(f), 0.0, f).astype(np.float32)
    codes, scales = oracle.quantize_int8(clean, "f32")
    codes[bad] = np.int8(0x5A)
    scales = scales.copy()
    scales[bad] = np.nan
    return codes, scales


def _run(wl, dtype_q, block_table=None, expect_error=0):
    import paged_kv_cache_61_amd as pkv
    bt = wl.block_table if block_table is None else block_table
    codes, scales = _quantised_pool(wl)
    d_codes = torch.from_numpy(codes).cuda()
    d_scales = scales_to_dev(scales)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.paged_kv_write_int8(to_dev(wl.k_new, wl.dtype), to_dev(wl.v_new, wl.dtype),
                            torch.from_numpy(wl.slot_mapping).cuda(), d_codes, d_scales, device_error=err)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    ws = torch.empty(max(256, pkv.paged_attention_workspace_size(wl.num_reqs, wl.num_tokens, wl.num_q_heads,
                                                                 wl.head_dim, wl.max_query_len, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = pkv.paged_attention_int8(to_dev(wl.q, dtype_q), d_codes, d_scales, i32(bt),
                                   i32(wl.seq_lens), i32(wl.query_start_loc), i32(wl.num_computed_tokens),
                                   wl.scale, max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                                   workspace=ws)
    again = pkv.paged_attention_int8(to_dev(wl.q, dtype_q), d_codes, d_scales, i32(bt),
                                     i32(wl.seq_lens), i32(wl.query_start_loc), i32(wl.num_computed_tokens),
                                     wl.scale, max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and pkv.pkv_read_device_error(ws) == expect_error
    # deterministic: the same bits (NaN rows included)
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       again.view(torch.int16) if again.dtype == torch.bfloat16 else again.view(torch.int32))
    ref_codes, ref_scales = oracle.kv_write_int8(codes, scales, wl.k_new, wl.v_new, wl.slot_mapping, wl.dtype)
    return out, d_codes.cpu().numpy(), scales_from_dev(d_scales), ref_codes, ref_scales


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 8, 8), ("bf16", 128, 32, 8), ("bf16", 64, 16, 2),
                                            ("f32", 64, 8, 2), ("f32", 128, 4, 4), ("bf16", 128, 64, 8),
                                            ("bf16", 128, 16, 1), ("bf16", 64, 32, 2), ("bf16", 128, 6, 2),
                                            ("f32", 128, 16, 2)])
def test_int8_write_and_attention(dtype, D, Hq, Hkv):
    _gpu()
    reqs = [(0, 1), (37, 1), (600, 1), (1500, 1), (15, 9), (40, 33), (0, 70), (511, 1), (512, 1), (2100, 2)]
    wl = workloads.build(workloads.small_spec(f"int8 {dtype} {D} {Hq}/{Hkv}", 31, dtype, Hq, Hkv, D, reqs))
    out, got_codes, got_scales, ref_codes, ref_scales = _run(wl, dtype)
    # write: bit for bit (NaN scales of untouched slots compared as bits)
    assert np.array_equal(got_codes, ref_codes)
    assert got_scales.tobytes() == ref_scales.astype(np.float32).tobytes()
    ref = oracle.attention_int8(wl.q, ref_codes, np.nan_to_num(ref_scales, nan=0.0), wl.block_table,
                                wl.seq_lens, wl.query_start_loc, wl.num_computed_tokens, wl.scale, dtype)
    assert_close(out_f64(out), ref, dtype, f"int8 cache attention {D} {Hq}/{Hkv}")
    # for information: distance from attention over the unquantised cache
    plain = oracle.attention(wl.q, oracle.kv_write(wl.pool, wl.k_new, wl.v_new, wl.slot_mapping), wl.block_table,
                             wl.seq_lens, wl.query_start_loc, wl.num_computed_tokens, wl.scale, dtype)
    print(f"[int8] quantisation effect on the output: max abs {np.abs(out_f64(out) - plain).max():.4f}", flush=True)


@pytest.mark.parametrize("Hq,Hkv,neg", [(32, 8, False), (8, 8, False), (64, 8, False), (16, 1, True),
                                         (8, 2, False)])
def test_int8_prefill_chunks_on_matrix_cores(Hq, Hkv, neg):
    # bf16 q, head_dim 128: prefill chunks run on the MFMA kernel, which
    # dequantises the streamed int8 tiles in LDS.  Chunks of many 64-key
    # tiles (the int8 ring and both dequantised K/V buffers wrap), ragged
    # tails, a prefix past 8192 keys (ids read per tile), a negative scale.
    _gpu()
    reqs = [(1000, 300), (0, 517), (3000, 64), (130, 1), (8200, 40), (63, 65), (5, 2)]
    wl = workloads.build(workloads.small_spec(f"int8 prefill {Hq}/{Hkv}", 57, "bf16", Hq, Hkv, 128, reqs))
    if neg:
        wl.scale = -wl.scale
    out, _, _, ref_codes, ref_scales = _run(wl, "bf16")
    ref = oracle.attention_int8(wl.q, ref_codes, np.nan_to_num(ref_scales, nan=0.0), wl.block_table,
                                wl.seq_lens, wl.query_start_loc, wl.num_computed_tokens, wl.scale, "bf16")
    assert_close(out_f64(out), ref, "bf16", f"int8 prefill {Hq}/{Hkv} neg={neg}")


def test_int8_prefill_bad_block_id_confined_to_its_request():
    # an id outside the pool in a chunk's table (in the first 128 tiles of
    # one request, past them in another) is reported and turns only those
    # requests' rows into NaN
    _gpu()
    import paged_kv_cache_61_amd as pkv
    reqs = [(9000, 70), (500, 100), (20, 1), (300, 50), (2000, 1)]
    wl = workloads.build(workloads.small_spec("int8 prefill bad id", 58, "bf16", 16, 4, 128, reqs))
    good, *_ = _run(wl, "bf16")
    bt = wl.block_table.copy()
    bt[0, 4 * 130 + 1] = wl.num_blocks + 3
    bt[1, 5] = -2
    bt[4, 70] = wl.num_blocks + 9     # a decode row: the second of its two 1024-token partitions
    out, *_ = _run(wl, "bf16", block_table=bt, expect_error=pkv.DEVERR_BLOCK_ID)
    o, gd = out_f64(out), out_f64(good)
    assert np.isnan(o[0:170]).all() and np.isnan(o[221]).all()
    assert np.array_equal(o[170:221], gd[170:221])


def test_int8_write_zero_rows_and_padding():
    _gpu()
    import paged_kv_cache_61_amd as pkv
    T, Hkv, D, NB = 6, 2, 128, 4
    rng = np.random.default_rng(3)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    k[1] = 0.0                      # all-zero rows: scale 0, codes 0
    v[2, 1] = 0.0
    slots = np.array([3, 17, -1, 40, 63, 0], np.int64)   # one padding token
    codes = np.full((2, NB, 16, Hkv, D), 7, np.int8)
    scales = np.full((2, NB, 16, Hkv), 5.0, np.float32)
    d_codes, d_scales = torch.from_numpy(codes).cuda(), scales_to_dev(scales)
    pkv.paged_kv_write_int8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda(),
                            d_codes, d_scales)
    torch.cuda.synchronize()
    rc, rs = oracle.kv_write_int8(codes, scales, k, v, slots, "f32")
    assert np.array_equal(d_codes.cpu().numpy(), rc) and scales_from_dev(d_scales).tobytes() == rs.tobytes()
    assert rs[0, 1, 1].tolist() == [0.0, 0.0]


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("dtype,D,Hkv,T", [("bf16", 64, 3, 37), ("bf16", 128, 3, 1000), ("f32", 128, 1, 7),
                                           ("f32", 64, 5, 513)])
def test_8bit_write_ragged_rows_and_bad_slots(fmt, dtype, D, Hkv, T):
    # the write kernel spreads a row over head_dim/8 lanes and takes row sets
    # of 64/(head_dim/8) rows, several per wave: row counts that leave the
    # last set partly empty, a padding token and two out-of-range slots (not
    # written, reported), everything else bit for bit as the oracle
    _gpu()
    import paged_kv_cache_61_amd as pkv
    NB = (T + 15) // 16 + 3
    print(f"[case] 8-bit write {fmt} {dtype} D={D} Hkv={Hkv} T={T}", flush=True)
    g = torch.Generator().manual_seed(T * 7 + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kt = torch.randn((T, Hkv, D), generator=g).to(tdt)
    vt = torch.randn((T, Hkv, D), generator=g).to(tdt)
    k, v = kt.float().numpy(), vt.float().numpy()   # the stored values, exactly
    rng = np.random.default_rng(T + D)
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    slots[T // 2] = -1                               # padding token
    bad = [T - 1, 0] if T > 2 else [T - 1]
    slots[bad[0]] = NB * 16 + 5                      # past the pool
    if len(bad) > 1:
        slots[bad[1]] = -7                           # negative, not -1
    cdt = np.int8 if fmt == "int8" else np.uint8
    codes = np.full((2, NB, 16, Hkv, D), 7, cdt)
    scales = np.full((2, NB, 16, Hkv), 5.0, np.float32)
    d_codes, d_scales = torch.from_numpy(codes).cuda(), scales_to_dev(scales)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    write = pkv.paged_kv_write_int8 if fmt == "int8" else pkv.paged_kv_write_fp8
    write(kt.cuda(), vt.cuda(), torch.from_numpy(slots).cuda(), d_codes, d_scales, device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & pkv.DEVERR_SLOT
    ok_slots = slots.copy()
    ok_slots[bad] = -1                               # the oracle skips them
    quant = oracle.kv_write_int8 if fmt == "int8" else oracle.kv_write_fp8
    rc, rs = quant(codes, scales, k, v, ok_slots, "f32")
    assert np.array_equal(d_codes.cpu().numpy(), rc)
    assert scales_from_dev(d_scales).tobytes() == rs.tobytes()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n,all_rows", [(2, True), (4, False), (5, True)])
def test_int8_workload_full_size(n, all_rows):
    # the benchmark's decode, mixed-step and long-context (32 split-KV
    # partitions per row) workloads at full size: every row of the decode
    # workloads, sampled rows of the mixed step
    _gpu()
    from gpu_util import eightbit_full
    eightbit_full("int8", n, 70 + n, all_rows=all_rows)
