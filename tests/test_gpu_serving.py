"""A short serving loop on the GPU: the host block manager schedules each
step (chunked prefills, decodes, prefix-cache hits, forks with copy-on-write),
the HIP path runs paged_kv_copy_blocks + paged_kv_write + paged_attention, and
every step is checked:

* the device cache equals the oracle's pool (block copies + writes) bit for
  bit, NaN sentinels of never-written slots included;
* each request's K/V read back through its block table equals the request's
  logical history (what a contiguous cache would hold);
* the attention output matches the fp64 oracle within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.block_manager as obm
import workloads
from gpu_util import TOL, assert_close, from_dev, out_f64, to_dev

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 8, 2, 128), ("f32", 4, 1, 64)])
def test_serving_loop_with_block_manager(dtype, Hq, Hkv, D):
    _gpu()
    import paged_kv_cache_61_amd as pkv
    NB, MB = 72, 12
    rng = np.random.default_rng(77)
    draw = lambda shape: (workloads.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))
                          if dtype == "bf16" else rng.standard_normal(shape).astype(np.float32))
    store = np.uint16 if dtype == "bf16" else np.float32
    nan = workloads.BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    host_pool = np.full((2, NB, 16, Hkv, D), nan, dtype=store)
    dev_pool = to_dev(host_pool, dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bm = pkv.BlockManager(NB, MB)
    ref_bm = obm.BlockManager(NB, MB)
    hist = {}                      # req id -> (K, V) storage arrays of the computed tokens
    live, nid = [], 1
    scale = 1.0 / np.sqrt(D)
    checked_rows = copies_seen = shared_seen = 0

    def add(rid, n, **kw):
        bm.add_request(rid, n, **kw)
        ref_bm.add_request(rid, n, **kw)
        nt, nc, _ = bm.request_state(rid)
        src = kw.get("prefix_from")
        hist[rid] = ((hist[src][0][:nc].copy(), hist[src][1][:nc].copy()) if nc else
                     (np.zeros((0, Hkv, D), store), np.zeros((0, Hkv, D), store)))
        live.append(rid)

    for step_no in range(14):
        # request traffic
        if step_no < 4 or rng.random() < 0.5:
            n = int(rng.choice([3, 16, 40, 75]))
            src = [r for r in live if bm.request_state(r)[1] >= 16]
            if src and rng.random() < 0.4:
                add(nid, n + 20, prefix_from=int(rng.choice(src)), prefix_tokens=int(rng.integers(16, 64)))
                shared_seen += 1
            else:
                add(nid, n)
            nid += 1
        done = [r for r in live if bm.request_state(r)[0] == bm.request_state(r)[1]]
        if done and rng.random() < 0.4:
            parent = int(rng.choice(done))
            bm.fork(parent, nid)
            ref_bm.fork(parent, nid)
            hist[nid] = (hist[parent][0].copy(), hist[parent][1].copy())
            live.append(nid)
            nid += 1
        for r in list(live):
            nt, nc, _ = bm.request_state(r)
            if nt == nc:
                if rng.random() < 0.15 and len(live) > 2:
                    bm.finish(r)
                    ref_bm.finish(r)
                    live.remove(r)
                else:
                    bm.append_tokens(r, 1)       # a sampled token to decode next
                    ref_bm.append_tokens(r, 1)

        st = bm.schedule(6, 96, MB * 16)
        ref = ref_bm.schedule(6, 96, MB * 16)
        for f in ("req_ids", "query_start_loc", "seq_lens", "num_computed_tokens", "block_table",
                  "slot_mapping", "copies"):
            assert np.array_equal(getattr(st, f), getattr(ref, f)), f
        T = st.num_tokens
        if T == 0:
            bm.commit()
            ref_bm.commit()
            continue
        k_new, v_new, q = draw((T, Hkv, D)), draw((T, Hkv, D)), draw((T, Hq, D))
        print(f"[serving] {dtype} step {step_no}: {st.num_reqs} reqs, {T} tokens, "
              f"{len(st.copies)} copies", flush=True)

        # device: copies, then the write, then attention (one stream)
        if len(st.copies):
            pkv.paged_kv_copy_blocks(dev_pool, torch.from_numpy(st.copies).cuda(), device_error=err)
            copies_seen += len(st.copies)
        pkv.paged_kv_write(to_dev(k_new, dtype), to_dev(v_new, dtype), torch.from_numpy(st.slot_mapping).cuda(),
                           dev_pool, device_error=err)
        # the table goes as scheduled, -1 in unused entries: a read of one
        # would set PKV_DEVERR_BLOCK_ID
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        ws = torch.empty(max(256, pkv.paged_attention_workspace_size(st.num_reqs, T, Hq, D, st.max_query_len,
                                                                     st.max_seq_len)),
                         dtype=torch.uint8, device="cuda")
        out = pkv.paged_attention(to_dev(q, dtype), dev_pool, i32(st.block_table), i32(st.seq_lens),
                                  i32(st.query_start_loc), i32(st.num_computed_tokens), scale,
                                  max_query_len=st.max_query_len, max_seq_len=st.max_seq_len, workspace=ws)
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and pkv.pkv_read_device_error(ws) == 0

        # oracle: the same copies and writes on the host pool
        host_pool = oracle.kv_write(oracle.copy_blocks(host_pool, st.copies), k_new, v_new, st.slot_mapping)
        assert from_dev(dev_pool).tobytes() == host_pool.tobytes(), f"cache differs at step {step_no}"
        # logical histories: append the step's new K/V and compare with the paged read-back
        for i, r in enumerate(st.req_ids.tolist()):
            a, b = int(st.query_start_loc[i]), int(st.query_start_loc[i + 1])
            hist[r] = (np.concatenate([hist[r][0], k_new[a:b]]), np.concatenate([hist[r][1], v_new[a:b]]))
            K, V = oracle.gather_kv(host_pool, st.block_table[i], int(st.seq_lens[i]), dtype)
            assert np.array_equal(K, oracle.to_f64(hist[r][0], dtype))
            assert np.array_equal(V, oracle.to_f64(hist[r][1], dtype))
        ref_out = oracle.attention(q, host_pool, np.where(st.block_table < 0, 0, st.block_table),
                                   st.seq_lens, st.query_start_loc, st.num_computed_tokens, scale, dtype)
        assert_close(out_f64(out), ref_out, dtype, f"serving step {step_no}")
        checked_rows += T
        bm.commit()
        ref_bm.commit()
    assert checked_rows > 200 and copies_seen >= 1 and shared_seen >= 1
