"""FP8 (OCP E4M3) KV cache on the GPU against the fp64 oracle.

* paged_kv_write_fp8: codes and scales bit for bit (both sides encode from
  the format's definition, on the same IEEE float32 quotient), untouched
  slots unchanged.
* The hardware decode of every finite code: a single-token context returns
  its V row exactly (softmax weight 1), so the output is the decoded V row
  times its scale, bit for bit, on the matrix-core row kernel (bf16 q), the
  VALU row kernel (fp32 q) and the prefill kernel (first row of a chunk).
* paged_attention_fp8: decode rows, prefill chunks and split-KV rows over the
  dequantised cache within the output tolerance, for bf16 and fp32 q, head_dim
  64 / 128 and several GQA groups; unused slots hold garbage codes and NaN
  scales, which must never reach the output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_close, out_f64, scales_from_dev, scales_to_dev, to_dev

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
    codes, scales = oracle.quantize_fp8(clean, "f32")
    codes[bad] = np.uint8(0x5A)
    scales = scales.copy()
    scales[bad] = np.nan
    return codes, scales


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _attend(wl, dtype_q, d_codes, d_scales, block_table=None):
    import paged_kv_cache_61_amd as pkv
    bt = wl.block_table if block_table is None else block_table
    ws = torch.empty(max(256, pkv.paged_attention_workspace_size(wl.num_reqs, wl.num_tokens, wl.num_q_heads,
                                                                 wl.head_dim, wl.max_query_len, wl.max_seq_len)),
                     dtype=torch.uint8, device="cuda")
    out = pkv.paged_attention_fp8(to_dev(wl.q, dtype_q), d_codes, d_scales, _i32(bt), _i32(wl.seq_lens),
                                  _i32(wl.query_start_loc), _i32(wl.num_computed_tokens), wl.scale,
                                  max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, workspace=ws)
    torch.cuda.synchronize()
    return out, pkv.pkv_read_device_error(ws)


def _run(wl, dtype_q, block_table=None, expect_error=0):
    import paged_kv_cache_61_amd as pkv
    codes, scales = _quantised_pool(wl)
    d_codes = torch.from_numpy(codes).cuda()
    d_scales = scales_to_dev(scales)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.paged_kv_write_fp8(to_dev(wl.k_new, wl.dtype), to_dev(wl.v_new, wl.dtype),
                           torch.from_numpy(wl.slot_mapping).cuda(), d_codes, d_scales, device_error=err)
    out, ws_err = _attend(wl, dtype_q, d_codes, d_scales, block_table)
    assert int(err.item()) == 0 and ws_err == expect_error
    again, _ = _attend(wl, dtype_q, d_codes, d_scales, block_table)     # deterministic: same bits
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       again.view(torch.int16) if again.dtype == torch.bfloat16 else again.view(torch.int32))
    ref_codes, ref_scales = oracle.kv_write_fp8(codes, scales, wl.k_new, wl.v_new, wl.slot_mapping, wl.dtype)
    return out, d_codes.cpu().numpy(), scales_from_dev(d_scales), ref_codes, ref_scales


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 8, 8), ("bf16", 128, 32, 8), ("bf16", 64, 16, 2),
                                            ("f32", 64, 8, 2), ("f32", 128, 4, 4), ("bf16", 128, 64, 8),
                                            ("bf16", 128, 16, 1), ("f32", 128, 16, 2)])
def test_fp8_write_and_attention(dtype, D, Hq, Hkv):
    _gpu()
    reqs = [(0, 1), (37, 1), (600, 1), (1500, 1), (15, 9), (40, 33), (0, 70), (511, 1), (512, 1), (2100, 2)]
    wl = workloads.build(workloads.small_spec(f"fp8 {dtype} {D} {Hq}/{Hkv}", 33, dtype, Hq, Hkv, D, reqs))
    out, got_codes, got_scales, ref_codes, ref_scales = _run(wl, dtype)
    # write: bit for bit (NaN scales of untouched slots compared as bits)
    assert np.array_equal(got_codes, ref_codes)
    assert got_scales.tobytes() == ref_scales.astype(np.float32).tobytes()
    ref = oracle.attention_fp8(wl.q, ref_codes, np.nan_to_num(ref_scales, nan=0.0), wl.block_table,
                               wl.seq_lens, wl.query_start_loc, wl.num_computed_tokens, wl.scale, dtype)
    assert_close(out_f64(out), ref, dtype, f"fp8 cache attention {D} {Hq}/{Hkv}")


@pytest.mark.parametrize("dtype,D,ql", [("bf16", 128, 1), ("f32", 128, 1), ("bf16", 64, 1), ("f32", 64, 1),
                                        ("bf16", 128, 2)])
def test_fp8_every_code_decodes_exactly(dtype, D, ql):
    # one request whose first query row sees only key 0: the output row is
    # V[0] decoded, times its scale (a power of two, so exact in bf16 too)
    _gpu()
    Hkv = 256 // D                 # 256 slots of V row 0: the 254 finite codes and two zeros
    Hq = 2 * Hkv
    wl = workloads.build(workloads.small_spec(f"fp8 codes {dtype} {D}", 34, dtype, Hq, Hkv, D, [(0, ql)]))
    codes, scales = _quantised_pool(wl)
    all_codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    rng = np.random.default_rng(35)
    blk = int(wl.block_table[0, 0])
    v_codes = np.concatenate([rng.permutation(all_codes), np.array([0x00, 0x80], np.uint8)]).reshape(Hkv, D)
    codes[1, blk, 0] = v_codes
    scales[1, blk, 0] = np.float32(0.25)
    codes[0, blk, 0] = rng.integers(0, 0x7E, (Hkv, D)).astype(np.uint8)
    scales[0, blk, 0] = np.float32(0.5)
    if ql > 1:   # the chunk's second key: any finite codes
        codes[:, blk, 1] = rng.integers(0, 0x7E, (2, Hkv, D)).astype(np.uint8)
        scales[:, blk, 1] = np.float32(1.0)
    out, err = _attend(wl, dtype, torch.from_numpy(codes).cuda(), scales_to_dev(scales))
    assert err == 0
    want = oracle.fp8_e4m3_decode(v_codes) * 0.25          # [Hkv, D]
    got = out_f64(out)[0].reshape(Hkv, Hq // Hkv, D)
    for g in range(Hkv):
        for h in range(Hq // Hkv):
            assert np.array_equal(got[g, h], want[g]), (g, h)
    # every code but the NaN pair appears
    assert set(np.unique(v_codes).tolist()) == set(all_codes.tolist())


@pytest.mark.parametrize("Hq,Hkv,neg", [(32, 8, False), (8, 8, False), (64, 8, False), (16, 1, True)])
def test_fp8_prefill_chunks_on_matrix_cores(Hq, Hkv, neg):
    # bf16 q, head_dim 128: prefill chunks on the MFMA kernel, which
    # dequantises the streamed tiles in LDS; long chunks, ragged tails, a
    # prefix past 8192 keys, a negative scale
    _gpu()
    reqs = [(1000, 300), (0, 517), (3000, 64), (130, 1), (8200, 40), (63, 65), (5, 2)]
    wl = workloads.build(workloads.small_spec(f"fp8 prefill {Hq}/{Hkv}", 59, "bf16", Hq, Hkv, 128, reqs))
    if neg:
        wl.scale = -wl.scale
    out, _, _, ref_codes, ref_scales = _run(wl, "bf16")
    ref = oracle.attention_fp8(wl.q, ref_codes, np.nan_to_num(ref_scales, nan=0.0), wl.block_table,
                               wl.seq_lens, wl.query_start_loc, wl.num_computed_tokens, wl.scale, "bf16")
    assert_close(out_f64(out), ref, "bf16", f"fp8 prefill {Hq}/{Hkv} neg={neg}")


def test_fp8_bad_block_id_confined_to_its_request():
    _gpu()
    import paged_kv_cache_61_amd as pkv
    reqs = [(9000, 70), (500, 100), (20, 1), (300, 50), (2000, 1)]
    wl = workloads.build(workloads.small_spec("fp8 bad id", 60, "bf16", 16, 4, 128, reqs))
    good, *_ = _run(wl, "bf16")
    bt = wl.block_table.copy()
    bt[0, 4 * 130 + 1] = wl.num_blocks + 3
    bt[1, 5] = -2
    bt[4, 70] = wl.num_blocks + 9     # a decode row: the second of its two 1024-token partitions
    out, *_ = _run(wl, "bf16", block_table=bt, expect_error=pkv.DEVERR_BLOCK_ID)
    o, gd = out_f64(out), out_f64(good)
    assert np.isnan(o[0:170]).all() and np.isnan(o[221]).all()
    assert np.array_equal(o[170:221], gd[170:221])


def test_fp8_write_zero_rows_negative_zero_and_padding():
    _gpu()
    import paged_kv_cache_61_amd as pkv
    T, Hkv, D, NB = 6, 2, 128, 4
    rng = np.random.default_rng(36)
    k = (rng.standard_normal((T, Hkv, D)) * rng.choice([1e-3, 1.0, 300.0], (T, Hkv, 1))).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    k[1] = 0.0                      # all-zero rows: scale 0, codes 0
    v[2, 1] = -0.0
    k[3, 0, :5] = -0.0              # negative zeros in a live row: code 0x80
    k[4, 1, 7] = k[4, 1].max() * 2  # a row max far above the rest: many subnormal codes
    slots = np.array([3, 17, -1, 40, 63, 0], np.int64)   # one padding token
    codes = np.full((2, NB, 16, Hkv, D), 7, np.uint8)
    scales = np.full((2, NB, 16, Hkv), 5.0, np.float32)
    d_codes, d_scales = torch.from_numpy(codes).cuda(), scales_to_dev(scales)
    pkv.paged_kv_write_fp8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda(),
                           d_codes, d_scales)
    torch.cuda.synchronize()
    rc, rs = oracle.kv_write_fp8(codes, scales, k, v, slots, "f32")
    assert np.array_equal(d_codes.cpu().numpy(), rc) and scales_from_dev(d_scales).tobytes() == rs.tobytes()
    assert rs[0, 1, 1].tolist() == [0.0, 0.0]
    assert (rc[0, 2, 8, 0, :5] == 0x80).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n,all_rows", [(2, True), (4, False), (5, True)])
def test_fp8_workload_full_size(n, all_rows):
    # the benchmark's decode, mixed-step and long-context (32 split-KV
    # partitions per row) workloads at full size: every row of the decode
    # workloads, sampled rows of the mixed step
    _gpu()
    from gpu_util import eightbit_full
    eightbit_full("fp8", n, 70 + n, all_rows=all_rows)
