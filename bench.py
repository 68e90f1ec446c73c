#!/usr/bin/env python3
"""Benchmark of one continuous-batching step of attention over a paged KV cache.

A step is the whole hot path over one batch: ``paged_kv_write`` of the step's
new tokens, then ``paged_attention`` (device-side planning, prefill chunks on
MFMA, decode rows with split-KV partitions, the split-KV merge, the output).
Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]

Default workload: the mixed continuous-batching step, bf16, token budget 8192
(3 chunked prefills of 2048 tokens on 0 / 1024 / 4096 cached tokens plus 2048
decode requests with contexts uniform in [256, 2048]; 32 q / 8 kv heads,
head_dim 128), the one workload that carries both halves of the metric:
decode KV-read GB/s against HBM and prefill TFLOP/s against bf16 MFMA.
``--workload 2`` is the Llama-7B-shaped decode (64 sequences, 32/32 heads),
3 the GQA decode at 256 sequences, 5 the long-context split-KV decode.
Prints ONE JSON line.  Only one GPU is supported: ``--gpus`` above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
METRIC = "paged decode KV-read GB/s (% HBM peak); prefill attn TFLOPS (% MFMA)"
WORKLOAD_NAMES = {
    1: "tiny paged decode fp32",
    2: "Llama-7B-shaped single-layer decode bf16",
    3: "GQA decode at high concurrency bf16",
    4: "mixed continuous-batching step bf16",
    5: "long-context split-KV decode bf16",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-int8", action="store_true",
                    help="INT8 KV cache (paged_kv_write_int8 + paged_attention_int8)")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="FP8 (E4M3) KV cache (paged_kv_write_fp8 + paged_attention_fp8)")
    ap.add_argument("--no-staging", action="store_true",
                    help="8-bit caches: no staging area (the prefill dequantises every tile it streams)")
    ap.add_argument("--rope", action="store_true",
                    help="write the step's tokens with paged_kv_write_rope (RoPE on K, and on q in place)")
    ap.add_argument("--head-dim", type=int, choices=(64, 128), default=None,
                    help="run the workload at this head_dim instead of its own (same lengths and heads)")
    ap.add_argument("--no-peak-probes", action="store_true",
                    help="skip the measured-peak probes (a device copy and a bf16 GEMM)")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="CPU seconds the oracle baseline may spend on its sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain device-to-device copy of known size instead (HBM calibration)")
    ap.add_argument("--copy-gib", type=float, default=4.0)
    ap.add_argument("--block-manager", action="store_true",
                    help="time the host block manager building the mixed step's metadata instead (CPU only)")
    return ap.parse_args()


def accounting(wl):
    """Algorithmic work of one step (what the method must move / compute)."""
    import numpy as np
    s = 2 if wl.dtype == "bf16" else 4
    Hq, Hkv, D = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    ql = wl.query_lens.astype(np.int64)
    L = wl.seq_lens.astype(np.int64)
    c = wl.num_computed_tokens.astype(np.int64)
    dec = ql == 1
    pre = ql > 1
    kv_token_bytes = 2 * Hkv * D * s
    a = {}
    a["decode_rows"] = int(dec.sum())
    a["decode_kv_tokens"] = int(L[dec].sum())
    a["decode_kv_bytes"] = int(L[dec].sum()) * kv_token_bytes
    a["decode_io_bytes"] = 2 * int(dec.sum()) * Hq * D * s            # q read + out written
    a["decode_table_bytes"] = int(((L[dec] + 15) // 16).sum()) * 4
    a["decode_bytes"] = a["decode_kv_bytes"] + a["decode_io_bytes"] + a["decode_table_bytes"]
    # INT8 cache: one byte per element plus a float32 scale per (token, kv head) row
    a["decode_kv_bytes_int8"] = int(L[dec].sum()) * 2 * Hkv * (D + 4)
    a["decode_bytes_int8"] = a["decode_kv_bytes_int8"] + a["decode_io_bytes"] + a["decode_table_bytes"]
    a["prefill_pairs_per_head"] = int((ql[pre] * c[pre] + ql[pre] * (ql[pre] + 1) // 2).sum())
    a["prefill_flops"] = 4 * D * Hq * a["prefill_pairs_per_head"]
    a["prefill_bytes"] = int(L[pre].sum()) * kv_token_bytes + 2 * int(ql[pre].sum()) * Hq * D * s
    T = wl.num_tokens
    a["write_bytes"] = 2 * (2 * T * Hkv * D * s) + 8 * T
    a["write_rope_bytes"] = a["write_bytes"] + 2 * T * Hq * D * s + 8 * T + T * D * 4  # + q in/out, positions, cos/sin
    a["step_bytes"] = a["decode_bytes"] + a["prefill_bytes"] + a["write_bytes"]
    return a


def cpu_baseline(wl, acct, budget_s):
    """Time the fp64 oracle, as it stands, on a bounded sample of the same step.

    The sample is cut into independent pieces (a decode request, or a run of
    64 consecutive rows of a prefill chunk) that run on a pool of host threads,
    one BLAS thread each, until about ``budget_s`` seconds of wall time are
    spent.  Decode pieces are scaled to the step by KV tokens read, prefill
    pieces by algorithmic FLOPs; the step time estimated from both is reported
    in the unit of the step's ``value`` (algorithmic bytes per second).  The
    oracle's cache write is not timed: it returns a fresh copy of the whole
    pool (a property of its plain form, not of the write)."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    threads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                         else (os.cpu_count() or 1)))
    rng = np.random.default_rng(1234)
    ql = wl.query_lens
    qsl = wl.query_start_loc
    D, Hq = wl.head_dim, wl.num_q_heads
    pieces = []                                # (kind, tokens, work)
    dec = [int(r) for r in rng.permutation(np.nonzero(ql == 1)[0])]
    pre = [int(r) for r in np.nonzero(ql > 1)[0]]
    runs = []
    for r in pre:                             # runs of 64 rows at random places of each chunk
        c = int(wl.num_computed_tokens[r])
        for i0 in rng.permutation(np.arange(0, int(ql[r]), 64)):
            toks = list(range(int(qsl[r]) + int(i0), min(int(qsl[r]) + int(i0) + 64, int(qsl[r + 1]))))
            flops = sum(4 * D * Hq * (c + t - int(qsl[r]) + 1) for t in toks)
            runs.append(("prefill", toks, flops))
    runs = [runs[i] for i in rng.permutation(len(runs))]
    # interleave so a bounded run samples both kinds in proportion to their cost
    di = 0
    for run in runs:
        pieces.append(run)
        for _ in range(max(1, len(dec) // max(1, len(runs)))):
            if di < len(dec):
                pieces.append(("decode", [int(qsl[dec[di]])], int(wl.seq_lens[dec[di]])))
                di += 1
    pieces += [("decode", [int(qsl[r])], int(wl.seq_lens[r])) for r in dec[di:]]
    # the step's tokens placed in the host pool in place (the oracle's own
    # write returns a copy of the whole pool, which is not the write's cost)
    sm = wl.slot_mapping
    live = sm >= 0
    pool = wl.pool
    pool[0, sm[live] // 16, sm[live] % 16] = wl.k_new[live]
    pool[1, sm[live] // 16, sm[live] % 16] = wl.v_new[live]

    def one(piece):
        kind, toks, work = piece
        t = time.perf_counter()
        oracle.attention_rows(wl.q, pool, wl.block_table, wl.seq_lens, qsl, wl.num_computed_tokens,
                              wl.scale, wl.dtype, tokens=toks, max_run=64)
        return kind, work, time.perf_counter() - t

    done = {"decode": [0, 0.0, 0], "prefill": [0, 0.0, 0]}    # work, thread-seconds, pieces
    t0 = time.perf_counter()
    with threadpool_limits(1), cf.ThreadPoolExecutor(threads) as ex:
        it = iter(pieces)
        live = set()
        for _ in range(threads):
            p_ = next(it, None)
            if p_ is not None:
                live.add(ex.submit(one, p_))
        while live:
            fin, live = cf.wait(live, return_when=cf.FIRST_COMPLETED)
            for f in fin:
                kind, work, dt = f.result()
                done[kind][0] += work
                done[kind][1] += dt
                done[kind][2] += 1
            if time.perf_counter() - t0 < budget_s:
                for _ in fin:
                    p_ = next(it, None)
                    if p_ is not None:
                        live.add(ex.submit(one, p_))
    wall = time.perf_counter() - t0
    busy = done["decode"][1] + done["prefill"][1]
    # thread-seconds per unit of work, spread over the threads that ran
    est = 0.0
    parts = {}
    if acct["decode_rows"] and done["decode"][0]:
        per_tok = done["decode"][1] / done["decode"][0]
        t_dec = per_tok * acct["decode_kv_tokens"] / threads
        est += t_dec
        parts["decode_GB/s"] = round(acct["decode_bytes"] / t_dec / 1e9, 4)
    if acct["prefill_flops"] and done["prefill"][0]:
        per_flop = done["prefill"][1] / done["prefill"][0]
        t_pf = per_flop * acct["prefill_flops"] / threads
        est += t_pf
        parts["prefill_TFLOP/s"] = round(acct["prefill_flops"] / t_pf / 1e12, 6)
    step_bytes = acct["decode_bytes"] + acct["prefill_bytes"]
    return {"value": round(step_bytes / est / 1e9, 4) if est > 0 else None, "unit": "GB/s",
            "cores": threads, "kind": "oracle", **parts,
            "estimated_step_s": round(est, 3),
            "sample": f"{done['decode'][2]} decode requests and {done['prefill'][2]} prefill runs of <= 64 rows "
                      f"(seeded random order) in {wall:.1f} s on {threads} threads ({busy:.1f} thread-s); "
                      "numpy fp64 oracle, one BLAS thread per worker; per-KV-token and per-FLOP costs scaled "
                      "to the whole step (attention only; the cache write is not timed)",
            "host": platform.processor() or platform.machine(), "host_cpus": os.cpu_count()}


def copy_probe(args):
    """A plain copy kernel of known size: the practical HBM rate, and the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = int(args.copy_gib * (1 << 30)) // 4
    src = torch.randn(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    nbytes = 2 * n * 4
    print(json.dumps({"probe": "device copy (torch copy_)", "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
                      "frac_of_8TBs": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}), flush=True)


def block_manager_probe(args):
    """Host cost of the C++ block manager (pkv_bm_*) for the mixed continuous-
    batching step's shape: 2048 running decodes with contexts U[256, 2048]
    plus 3 new 2048-token prompts (one sharing a 256-token prefix), token
    budget 8192.  Times one pkv_bm_schedule + pkv_bm_commit pair per step (the
    C calls only, outputs preallocated), after the appends of the step's
    generated tokens."""
    import ctypes
    import time
    import numpy as np
    import paged_kv_cache_61_amd as pkv
    lib = pkv._lib
    NB, MB, S, BUDGET, MAXLEN = 200000, 512, 2051 + 8, 8192, 8192
    bm = pkv.BlockManager(NB, MB)
    rng = np.random.default_rng(4)
    for r, L in enumerate(rng.integers(256, 2049, 2048)):
        bm.add_request(r, int(L))
    while True:   # prefill every prompt (chunked) so the 2048 requests are decoding
        st = bm.schedule(S, BUDGET, MAXLEN)
        bm.commit()
        if st.max_query_len <= 1:
            break
    buf = dict(req_ids=np.zeros(S, np.int64), qsl=np.zeros(S + 1, np.int32), sl=np.zeros(S, np.int32),
               nct=np.zeros(S, np.int32), bt=np.zeros((S, MB), np.int32), sm=np.zeros(BUDGET, np.int64),
               cp=np.zeros((S, 2), np.int32))
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    step = pkv._PkvStep(S, BUDGET, MAXLEN, p(buf["req_ids"]), p(buf["qsl"]), p(buf["sl"]), p(buf["nct"]),
                        p(buf["bt"]), p(buf["sm"]), p(buf["cp"]), 0, 0, 0, 0, 0)
    times, kinds = [], []
    nxt = 2048
    for it in range(args.warmup + args.steps):
        for r in range(2048):
            bm.append_tokens(r, 1)
        if it % 8 == 0:   # new prompts arrive: three 2048-token requests, one with a shared prefix
            bm.add_request(nxt, 2048)
            bm.add_request(nxt + 1, 2048, prefix_from=0, prefix_tokens=256)
            bm.add_request(nxt + 2, 2048)
            new = [nxt, nxt + 1, nxt + 2]
            nxt += 3
        t0 = time.perf_counter()
        rc = lib.pkv_bm_schedule(bm._h, ctypes.byref(step))
        rc |= lib.pkv_bm_commit(bm._h)
        dt = time.perf_counter() - t0
        if rc != 0:
            raise SystemExit(f"block manager call failed: {rc}")
        if it % 8 == 7:
            for r in new:
                bm.finish(r)
        if it >= args.warmup:
            times.append(dt)
            kinds.append(step.max_query_len > 1)
    t = np.array(times) * 1e6
    mixed = t[np.array(kinds)] if any(kinds) else t
    print(json.dumps({"probe": "host block manager: pkv_bm_schedule + pkv_bm_commit per step",
                      "requests": int(step.num_reqs), "step_tokens": int(step.num_tokens),
                      "us_per_step_median": round(float(np.median(t)), 1),
                      "us_per_mixed_step_median": round(float(np.median(mixed)), 1),
                      "us_per_step_max": round(float(t.max()), 1), "steps": len(t)}), flush=True)


def row_kernel_name(wl, kv8):
    """The library kernel that runs the decode rows of this workload (kv8:
    None, "int8" or "fp8")."""
    if kv8:
        f = kv8.upper()
        return (f"row_attn_i8_mfma_kernel ({f} cache, bf16 q: decode rows + split-KV partitions)"
                if wl.dtype == "bf16" else f"row_attn_i8_kernel ({f} cache, fp32 q: decode rows + split-KV partitions)")
    g = wl.num_q_heads // wl.num_kv_heads
    if wl.dtype == "bf16" and (g > 4 or (g > 2 and wl.head_dim == 128)):
        return "row_attn_mfma_kernel (decode rows + split-KV partitions, all query heads of a kv head on MFMA)"
    return "row_attn_kernel (decode rows + split-KV partitions)"


WORKLOAD_TAGS = {2: "decode_llama7b_bs64", 3: "decode_gqa_bs256", 4: "mixed_step_8192",
                 5: "decode_long_context_g8"}


def measured_traffic(workload, role):
    """HBM bytes per launch of the ``role`` kernel ("rows" or "prefill") from the
    committed PMC record of this workload, if it was taken on the kernel's
    current source; else None."""
    import hashlib
    tag = WORKLOAD_TAGS.get(workload)
    if tag is None:
        return None
    rec_path = os.path.join(ROOT, "profiles", f"{tag}_traffic.json")
    if not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path)).get("kernels", {}).get(role)
    if not rec:
        return None
    src_path = os.path.join(ROOT, "paged_kv_cache_61_amd", "csrc", rec["source"])
    if hashlib.sha256(open(src_path, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes_per_launch"])


def peak_probes():
    """Measured ceilings on this GPU: a device-to-device copy (torch copy_,
    2 GiB each way) and a dense bf16 GEMM (torch.matmul, 8192^3, hipBLASLt)."""
    import torch
    res = {}
    n = (2 << 30) // 4
    src = torch.empty(n, device="cuda", dtype=torch.float32).fill_(1.0)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    for name, fn, work in (("copy_GB/s", lambda: dst.copy_(src), 2 * n * 4 / 1e9),
                           ("bf16_gemm_TFLOP/s", lambda: torch.matmul(a, b), 2 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(work / (e0.elapsed_time(e1) / 10 * 1e-3), 1)
    del src, dst, a, b
    torch.cuda.empty_cache()
    return res


def pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs), q)), 5)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args)
        return
    if args.block_manager:
        block_manager_probe(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.kv_int8 and args.kv_fp8:
        raise SystemExit("--kv-int8 and --kv-fp8 are separate modes")
    kv8 = "int8" if args.kv_int8 else "fp8" if args.kv_fp8 else None

    import numpy as np
    import torch

    import paged_kv_cache_61_amd as pkv
    import workloads

    t_gen = time.perf_counter()
    spec = workloads.BENCH_WORKLOADS[args.workload]
    if args.head_dim is not None and args.head_dim != spec.head_dim:
        import dataclasses
        spec = dataclasses.replace(spec, head_dim=args.head_dim,
                                   name=spec.name.replace("D=128", f"D={args.head_dim}") + f", head_dim {args.head_dim}")
    wl = workloads.build(spec)
    gen_s = time.perf_counter() - t_gen
    acct = accounting(wl)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    q, pool = up(wl.q), up(wl.pool)
    k_new, v_new = up(wl.k_new), up(wl.v_new)
    slot_mapping = torch.from_numpy(wl.slot_mapping).to(dev)
    bt, sl, qsl, nct = (i32(wl.block_table), i32(wl.seq_lens), i32(wl.query_start_loc),
                        i32(wl.num_computed_tokens))
    ws_bytes = pkv.paged_attention_workspace_size(wl.num_reqs, wl.num_tokens, wl.num_q_heads, wl.head_dim,
                                                  wl.max_query_len, wl.max_seq_len)
    stage_blocks = 0
    if kv8 and not args.no_staging:
        # 8-bit cache: room to stage the step's prefill blocks (dequantised once per step)
        ql = wl.query_lens
        stage_blocks = int(sum((int(wl.seq_lens[r]) + 15) // 16 for r in np.nonzero(ql > 1)[0]))
        ws_bytes += pkv.paged_attention_staging_bytes(wl.num_reqs, wl.block_table.shape[1], wl.num_kv_heads,
                                                      wl.head_dim, stage_blocks)
    ws = torch.empty(max(256, ws_bytes), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    nph = pkv.NUM_PHASES
    step_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nph + 2)]
                   for _ in range(args.steps)]
    if args.rope:
        positions = torch.from_numpy(np.concatenate(
            [np.arange(int(wl.num_computed_tokens[r]), int(wl.seq_lens[r])) for r in range(wl.num_reqs)]
        ).astype(np.int64)).to(dev)
        inv = 10000.0 ** (-np.arange(0, wl.head_dim, 2, dtype=np.float64) / wl.head_dim)
        ang = np.arange(wl.max_seq_len + 1, dtype=np.float64)[:, None] * inv[None, :]
        cos_sin = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).to(dev)
    for evs in step_events:          # create the underlying hipEvents
        for e in evs:
            e.record()
    torch.cuda.synchronize()

    if kv8:
        if args.rope:
            raise SystemExit("--kv-int8 / --kv-fp8 and --rope are separate modes")
        write8 = pkv.paged_kv_write_int8 if kv8 == "int8" else pkv.paged_kv_write_fp8
        attend8 = pkv.paged_attention_int8 if kv8 == "int8" else pkv.paged_attention_fp8
        # quantise every slot of the pool once (unused slots hold NaN: their
        # codes and scales are never read)
        nb = pool.shape[1]
        codes = torch.empty(pool.shape, dtype=torch.int8 if kv8 == "int8" else torch.uint8, device=dev)
        kv_scales = torch.empty((2, nb, wl.num_kv_heads, 16), dtype=torch.float32, device=dev)
        write8(pool[0].reshape(nb * 16, wl.num_kv_heads, wl.head_dim).contiguous(),
               pool[1].reshape(nb * 16, wl.num_kv_heads, wl.head_dim).contiguous(),
               torch.arange(nb * 16, dtype=torch.int64, device=dev), codes, kv_scales)
        del pool
        torch.cuda.synchronize()

    def step(evs=None):
        if evs is not None:
            evs[2 * nph].record()
        if kv8:
            write8(k_new, v_new, slot_mapping, codes, kv_scales)
            if evs is not None:
                evs[2 * nph + 1].record()
            attend8(q, codes, kv_scales, bt, sl, qsl, nct, wl.scale,
                    max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, out=out,
                    workspace=ws, phase_events=None if evs is None else evs[:2 * nph])
            return
        if args.rope:
            pkv.paged_kv_write_rope(k_new, v_new, positions, cos_sin, slot_mapping, pool, q=q)
        else:
            pkv.paged_kv_write(k_new, v_new, slot_mapping, pool)
        if evs is not None:
            evs[2 * nph + 1].record()
        pkv.paged_attention(q, pool, bt, sl, qsl, nct, wl.scale, max_query_len=wl.max_query_len,
                            max_seq_len=wl.max_seq_len, out=out, workspace=ws,
                            phase_events=None if evs is None else evs[:2 * nph])

    probes = None if args.no_peak_probes else peak_probes()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    err = pkv.pkv_read_device_error(ws)
    if err != 0:
        raise SystemExit(f"device error word {err:#x}")

    # Timed region 1: K plain steps (the library calls exactly as a caller
    # makes them) -> ms_per_step and the whole-step throughput.  An event
    # between steps gives the spread of single steps.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in marks:
        e.record()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    total_ms = marks[0].elapsed_time(marks[-1])
    ms_per_step = total_ms / args.steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    # Timed region 2: K more steps with hipEvents recorded by the library on
    # its own stream around each internal phase -> per-kernel launch times
    # (the events add a few microseconds per step, so region 1 gives the
    # step time).
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(step_events[i])
    torch.cuda.synchronize()
    names = ["plan", "prefill", "rows", "reduce"]
    phase_all = {nm: [evs[2 * p].elapsed_time(evs[2 * p + 1]) for evs in step_events]
                 for p, nm in enumerate(names)}
    phase_ms = {nm: float(np.mean(v)) for nm, v in phase_all.items()}

    write_ms = float(np.mean([evs[2 * nph].elapsed_time(evs[2 * nph + 1]) for evs in step_events]))
    write_bytes = acct["write_rope_bytes"] if args.rope else acct["write_bytes"]
    step_bytes = acct["step_bytes"] - acct["write_bytes"] + write_bytes
    dec_bytes = acct["decode_bytes"]
    if kv8:   # k/v read in their dtype, written as codes + scales
        T_, s_ = wl.num_tokens, 2 if wl.dtype == "bf16" else 4
        write_bytes = 2 * T_ * wl.num_kv_heads * (wl.head_dim * s_ + wl.head_dim + 4) + 8 * T_
        dec_bytes = acct["decode_bytes_int8"]
        step_bytes = dec_bytes + acct["prefill_bytes"] + write_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    rows_gbs = dec_bytes / (phase_ms["rows"] * 1e-3) / 1e9 if phase_ms["rows"] > 0 else 0.0
    roof_rows = {
        "kernel": row_kernel_name(wl, kv8),
        "bound": "hbm",
        "achieved": round(rows_gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(rows_gbs / HBM_PEAK_GBS, 4),
        "traffic": None if kv8 or args.head_dim not in (None, 128) else measured_traffic(args.workload, "rows"),
        "algorithmic_bytes_per_launch": dec_bytes,
        "avg_launch_ms": round(phase_ms["rows"], 5),
        "launch_ms_p10": pct(phase_all["rows"], 10), "launch_ms_p90": pct(phase_all["rows"], 90),
    }
    if probes:
        roof_rows["frac_of_measured_copy"] = round(rows_gbs / probes["copy_GB/s"], 4)
    roof_pf = None
    if acct["prefill_flops"] > 0 and phase_ms["prefill"] > 0.02:
        tf = acct["prefill_flops"] / (phase_ms["prefill"] * 1e-3) / 1e12
        roof_pf = {
            "kernel": "prefill_kernel (chunked prefill on bf16 MFMA"
                      + ((f", {kv8} cache dequantised once into a bf16 staging area; the phase includes the "
                          "staging kernel)" if stage_blocks else f", {kv8} cache dequantised in LDS)") if kv8 else ")"),
            "bound": "mfma",
            "achieved": round(tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None if kv8 or args.head_dim not in (None, 128) else measured_traffic(args.workload, "prefill"),
            "algorithmic_flops_per_launch": acct["prefill_flops"],
            "avg_launch_ms": round(phase_ms["prefill"], 5),
            "launch_ms_p10": pct(phase_all["prefill"], 10), "launch_ms_p90": pct(phase_all["prefill"], 90),
        }
        if probes:
            roof_pf["frac_of_measured_gemm"] = round(tf / probes["bf16_gemm_TFLOP/s"], 4)
    # the dominant kernel (longest launch) is the line's "roofline"
    dominant_is_pf = roof_pf is not None and phase_ms["prefill"] > phase_ms["rows"]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_ms_p10": pct(step_ms, 10), "step_ms_p50": pct(step_ms, 50), "step_ms_p90": pct(step_ms, 90),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, shuffled block pool, NaN-poisoned unused slots)",
        "config": {
            "workload": f"{WORKLOAD_NAMES[args.workload]}: {wl.spec.name}",
            "num_reqs": wl.num_reqs, "num_tokens": wl.num_tokens,
            "decode_rows": acct["decode_rows"], "prefill_rows": int(wl.num_tokens - acct["decode_rows"]),
            "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": 16, "num_blocks": wl.num_blocks,
            "decode_kv_tokens": acct["decode_kv_tokens"], "max_seq_len": wl.max_seq_len,
            "kv_cache": (f"{kv8} codes + float32 scale per (token, kv head)" if kv8 else wl.dtype),
            **({"prefill_staging_blocks": stage_blocks} if kv8 else {}),
        },
        "roofline": roof_pf if dominant_is_pf else roof_rows,
        "rooflines": {"decode_rows": roof_rows, **({"prefill": roof_pf} if roof_pf else {})},
        "phases_ms": {k: round(v, 5) for k, v in phase_ms.items()},
        "write": {"kernel": ("kv_write_rope_kernel (RoPE on K and q)" if args.rope else
                             f"kv_write_i8_kernel ({kv8} quantising)" if kv8 else "kv_write_kernel"),
                  "ms": round(write_ms, 5), "bytes": write_bytes,
                  "GB/s": round(write_bytes / (write_ms * 1e-3) / 1e9, 1) if write_ms > 0 else None},
        "step_algorithmic_bytes": step_bytes,
        "wall_s_timed": round(wall_s, 4),
        "input_gen_s": round(gen_s, 2),
    }
    if roof_pf:
        result["prefill_tflops"] = roof_pf["achieved"]
        result["prefill_frac_mfma_bf16"] = roof_pf["frac"]
        # the step against its two rooflines: bytes at 8 TB/s and FLOPs at 2.5 PFLOP/s
        t_mem = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        t_fl = acct["prefill_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
        result["step_vs_roofline"] = {"bytes_ms_at_peak": round(t_mem, 5), "flops_ms_at_peak": round(t_fl, 5),
                                      "measured_over_max": round(ms_per_step / max(t_mem, t_fl), 4),
                                      "measured_over_sum": round(ms_per_step / (t_mem + t_fl), 4)}
    result["decode_kv_read_GB/s"] = roof_rows["achieved"]
    result["decode_frac_hbm"] = roof_rows["frac"]
    if probes:
        result["measured_peaks"] = probes
    if not args.no_cpu_baseline and world == 1:
        result["cpu_baseline"] = cpu_baseline(wl, acct, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
