"""paged_attention_noalloc (workspace in the library's static device scratch)
against paged_attention (caller-owned workspace) through the C ABI: the same
inputs give the same bits, on two calls in a row, the second smaller than the
first, and device error bits reach the caller's int32."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import out_f64, run_attention, run_write, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(s, seq_lens=None):
    import paged_kv_cache_61_amd as pkv
    wl = s.wl
    out = torch.full_like(s.q, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.paged_attention_noalloc(s.q, s.pool, s.block_table, s.seq_lens if seq_lens is None else seq_lens,
                                s.qsl, s.nct, wl.scale, max_query_len=wl.max_query_len,
                                max_seq_len=wl.max_seq_len, out=out, device_error=err)
    torch.cuda.synchronize()
    return out, int(err.item())


def _bits(t):
    return t.detach().cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


# a mixed batch with MFMA prefill chunks and split-KV decode rows, then a
# smaller one; and fp32 (row-kernel prefill) the same way
CASES = [
    ("bf16", 32, 8, 128, [dict(num_reqs=48, max_ctx=5000, max_ql=700), dict(num_reqs=9, max_ctx=900, max_ql=40)]),
    ("f32", 8, 2, 64, [dict(num_reqs=20, max_ctx=2500, max_ql=60), dict(num_reqs=5, max_ctx=300, max_ql=20)]),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,sizes", CASES)
def test_noalloc_matches_paged_attention_on_two_calls(dtype, Hq, Hkv, D, sizes):
    for i, kw in enumerate(sizes):
        spec = workloads.random_spec(f"noalloc-{dtype}-{i}", 300 + i, dtype, Hq, Hkv, D, **kw)
        wl = workloads.build(spec)
        print(f"[case] {spec.name}: {wl.num_reqs} requests, {wl.num_tokens} tokens", flush=True)
        s = upload(wl)
        run_write(s)
        ref = run_attention(s).clone()
        torch.cuda.synchronize()
        got, err = _noalloc(s)
        assert err == 0
        assert np.array_equal(_bits(got), _bits(ref)), f"{spec.name}: outputs differ"


def test_noalloc_reports_device_errors_then_recovers():
    import paged_kv_cache_61_amd as pkv
    reqs = [(40, 1), (10, 3), (1200, 1)]
    wl = workloads.build(workloads.small_spec("noalloc-bad", 26, "bf16", 8, 2, 128, reqs))
    s = upload(wl)
    run_write(s)
    good = out_f64(run_attention(s))
    sl = s.seq_lens.clone()
    sl[1] += 1                                   # request 1 inconsistent
    out, err = _noalloc(s, seq_lens=sl)
    assert err & pkv.DEVERR_SEQ_LEN
    o = out_f64(out)
    assert np.isnan(o[1:4]).all()
    assert np.array_equal(o[[0, 4]], good[[0, 4]])
    out, err = _noalloc(s)                        # the next call starts clean
    assert err == 0
    assert np.array_equal(out_f64(out), good)
