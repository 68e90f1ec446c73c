"""Helpers for GPU parity tests: upload seeded workloads, run the HIP path
through the C ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": 1e-5, "bf16": 2e-2}


def to_dev(x: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Storage bits back to numpy (uint16 patterns for bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


@dataclasses.dataclass
class DevStep:
    wl: workloads.Workload
    q: torch.Tensor
    pool: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    qsl: torch.Tensor
    nct: torch.Tensor
    workspace: torch.Tensor
    out: torch.Tensor


def upload(wl: workloads.Workload) -> DevStep:
    import paged_kv_cache_61_amd as pkv
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    ws = pkv.paged_attention_workspace_size(wl.num_reqs, wl.num_tokens, wl.num_q_heads,
                                            wl.head_dim, wl.max_query_len, wl.max_seq_len)
    q = to_dev(wl.q, wl.dtype)
    return DevStep(wl=wl, q=q, pool=to_dev(wl.pool, wl.dtype), k_new=to_dev(wl.k_new, wl.dtype),
                   v_new=to_dev(wl.v_new, wl.dtype),
                   slot_mapping=torch.from_numpy(wl.slot_mapping).cuda(),
                   block_table=i32(wl.block_table), seq_lens=i32(wl.seq_lens),
                   qsl=i32(wl.query_start_loc), nct=i32(wl.num_computed_tokens),
                   workspace=torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda"),
                   out=torch.empty_like(q))


def run_write(s: DevStep) -> None:
    import paged_kv_cache_61_amd as pkv
    pkv.paged_kv_write(s.k_new, s.v_new, s.slot_mapping, s.pool)


def run_attention(s: DevStep, scale=None, out=None) -> torch.Tensor:
    import paged_kv_cache_61_amd as pkv
    wl = s.wl
    return pkv.paged_attention(s.q, s.pool, s.block_table, s.seq_lens, s.qsl, s.nct,
                               wl.scale if scale is None else scale,
                               max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                               out=s.out if out is None else out, workspace=s.workspace)


def device_error(s: DevStep) -> int:
    import paged_kv_cache_61_amd as pkv
    return pkv.pkv_read_device_error(s.workspace)


def oracle_pool(wl: workloads.Workload) -> np.ndarray:
    return oracle.kv_write(wl.pool, wl.k_new, wl.v_new, wl.slot_mapping)


def oracle_out(wl: workloads.Workload, pool: np.ndarray, tokens=None) -> np.ndarray:
    args = (wl.q, pool, wl.block_table, wl.seq_lens, wl.query_start_loc,
            wl.num_computed_tokens, wl.scale, wl.dtype)
    if tokens is None:
        return oracle.attention(*args)
    return oracle.attention_rows(*args, tokens=tokens)


def host_threads() -> int:
    """Worker threads for the oracle on the host: every CPU the process may
    use, at most 16 (the GPU machines give one GPU's job 16 CPUs)."""
    import os
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def oracle_rows_parallel(q: np.ndarray, pool: np.ndarray, wl: workloads.Workload, tokens, dtype: str,
                         chunk: int = 128) -> np.ndarray:
    """``oracle.attention_rows`` for ``tokens`` (sorted), cut into chunks of
    ``chunk`` rows that run on a pool of threads, each with one BLAS thread
    (the oracle's matrix products and exponentials release the GIL)."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    tokens = [int(t) for t in tokens]
    parts = [tokens[i:i + chunk] for i in range(0, len(tokens), chunk)]

    def one(part):
        return oracle.attention_rows(q, pool, wl.block_table, wl.seq_lens, wl.query_start_loc,
                                     wl.num_computed_tokens, wl.scale, dtype, tokens=part, max_run=chunk)
    with threadpool_limits(1), cf.ThreadPoolExecutor(host_threads()) as ex:
        res = list(ex.map(one, parts))
    return np.concatenate(res) if res else np.zeros((0,) + tuple(q.shape[1:]))


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    err = np.abs(got - ref)
    tol = TOL[dtype]
    stats = dict(max_abs=float(np.nanmax(err)) if err.size else 0.0,
                 mean_abs=float(np.nanmean(err)) if err.size else 0.0,
                 over=int((err > tol).sum()), nan=int(np.isnan(got).sum()))
    print(f"[parity] {what} {dtype}: {stats}", flush=True)
    assert stats["nan"] == 0 and not np.isnan(err).any(), f"{what}: NaN in output"
    assert stats["max_abs"] <= tol, f"{what}: max abs err {stats['max_abs']} > {tol}"
    return stats


def scales_to_dev(scales: np.ndarray) -> torch.Tensor:
    """Per-row scales in the oracle's cache order [2, NB, 16, Hkv] -> the
    library's 8-bit scale layout [2, NB, Hkv, 16] on the device."""
    return torch.from_numpy(np.ascontiguousarray(np.asarray(scales, np.float32).transpose(0, 1, 3, 2))).cuda()


def scales_from_dev(t: torch.Tensor) -> np.ndarray:
    """The inverse of scales_to_dev: [2, NB, Hkv, 16] -> [2, NB, 16, Hkv] (numpy)."""
    return np.ascontiguousarray(t.cpu().numpy().transpose(0, 1, 3, 2))


def _quantise_blocks_parallel(quant, pool_sub: np.ndarray, dtype: str, step: int = 1024):
    """The oracle's quantisation of ``pool_sub [2, nb, 16, Hkv, D]``, row by
    row (every (token, kv head) row is independent), in slices of blocks on a
    pool of threads."""
    import concurrent.futures as cf
    nb = pool_sub.shape[1]
    codes = np.empty(pool_sub.shape, np.int8 if quant is oracle.quantize_int8 else np.uint8)
    scales = np.empty(pool_sub.shape[:-1], np.float32)

    def one(lo):
        c, sc = quant(pool_sub[:, lo:lo + step], dtype)
        codes[:, lo:lo + step] = c
        scales[:, lo:lo + step] = sc
    with cf.ThreadPoolExecutor(host_threads()) as ex:
        list(ex.map(one, range(0, nb, step)))
    return codes, scales


def eightbit_full(fmt: str, n: int, seed: int, all_rows: bool = False) -> None:
    """An 8-bit cache (``fmt`` "int8" or "fp8") at a benchmark workload's full
    size, in the benchmark's launch configuration: the whole pool quantised on
    the device, the step's tokens written, one attention call.  The codes and
    scales of every block the checked rows read are compared bit for bit with
    the oracle's quantisation of the same (written) pool, and the checked rows
    with the oracle's attention over those dequantised blocks.  Checked rows:
    every row when ``all_rows``, else the first, last and random rows of each
    prefill chunk and 48 random decode rows."""
    import paged_kv_cache_61_amd as pkv
    write8 = pkv.paged_kv_write_int8 if fmt == "int8" else pkv.paged_kv_write_fp8
    attend8 = pkv.paged_attention_int8 if fmt == "int8" else pkv.paged_attention_fp8
    quant = oracle.quantize_int8 if fmt == "int8" else oracle.quantize_fp8
    deq = oracle.dequantize_int8 if fmt == "int8" else oracle.dequantize_fp8
    wl = workloads.build(workloads.BENCH_WORKLOADS[n])
    print(f"[case] {fmt} workload {n}: {wl.spec.name} ({'all rows' if all_rows else 'sampled rows'})",
          flush=True)
    s = upload(wl)
    NB, Hkv, D = wl.num_blocks, wl.num_kv_heads, wl.head_dim
    codes = torch.empty(tuple(s.pool.shape), dtype=torch.int8 if fmt == "int8" else torch.uint8, device="cuda")
    scales = torch.empty((2, NB, Hkv, 16), dtype=torch.float32, device="cuda")
    write8(s.pool[0].reshape(NB * 16, Hkv, D).contiguous(), s.pool[1].reshape(NB * 16, Hkv, D).contiguous(),
           torch.arange(NB * 16, dtype=torch.int64, device="cuda"), codes, scales)
    del s.pool
    write8(s.k_new, s.v_new, s.slot_mapping, codes, scales)
    attend8(s.q, codes, scales, s.block_table, s.seq_lens, s.qsl, s.nct, wl.scale,
            max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, out=s.out, workspace=s.workspace)
    torch.cuda.synchronize()
    assert device_error(s) == 0
    qsl, ql = wl.query_start_loc, np.diff(wl.query_start_loc)
    if all_rows:
        rows = list(range(wl.num_tokens))
    else:
        rng = np.random.default_rng(seed)
        rows = []
        for r in np.nonzero(ql > 1)[0][:4]:  # prefill chunks: first, last and random rows
            rows += [int(qsl[r]), int(qsl[r + 1]) - 1] + rng.integers(qsl[r], qsl[r + 1], 10).tolist()
        dec = np.nonzero(ql == 1)[0]
        rows += [int(qsl[r]) for r in rng.choice(dec, min(48, len(dec)), replace=False)]
        rows = sorted(set(rows))
    reqs = sorted({int(np.searchsorted(qsl, t, side="right") - 1) for t in rows})
    blocks = sorted({int(b) for r in reqs for b in wl.block_table[r, :(int(wl.seq_lens[r]) + 15) // 16]})
    ref_pool = oracle_pool(wl)[:, blocks]                         # [2, nsub, 16, Hkv, D]
    with np.errstate(invalid="ignore"):
        live = ~np.isnan(oracle.to_f64(ref_pool, wl.dtype)).any(axis=-1)   # unused slots are NaN
    rc, rs = _quantise_blocks_parallel(quant, np.where(live[..., None], ref_pool, 0).astype(ref_pool.dtype),
                                       wl.dtype)
    del ref_pool
    idx = torch.tensor(blocks, dtype=torch.int64, device="cuda")
    gc = codes.index_select(1, idx).cpu().numpy()
    gs = scales_from_dev(scales.index_select(1, idx))
    assert np.array_equal(gc[live], rc[live]), "codes differ"
    assert gs[live].tobytes() == rs[live].tobytes(), "scales differ"
    del gc, gs
    # attention over the dequantised blocks (block ids remapped to the subset)
    remap = np.full(NB, -1, np.int64)
    remap[blocks] = np.arange(len(blocks))
    bt = np.zeros_like(wl.block_table)
    for r in reqs:
        nb_r = (int(wl.seq_lens[r]) + 15) // 16
        bt[r, :nb_r] = remap[wl.block_table[r, :nb_r]]
    pool_deq = np.where(live[..., None], deq(rc, rs), 0.0)
    del rc, rs
    sub = dataclasses.replace(wl, block_table=bt)
    ref = oracle_rows_parallel(oracle.to_f64(wl.q, wl.dtype), pool_deq, sub, rows, "f64")
    assert_close(out_f64(s.out)[rows], ref, wl.dtype,
                 f"{fmt} workload {n} {'all rows' if all_rows else 'sampled'}")
