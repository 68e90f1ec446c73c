"""The C-ABI library on the CPU: it loads, exports what include/paged_kv.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "paged_kv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    import paged_kv_cache_61_amd as pkv
    names = _declared()
    assert {"paged_kv_write", "paged_attention", "paged_attention_workspace_size"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(pkv._lib, n)


def _attn(lib, **kw):
    a = dict(out=None, q=None, kv=16, bt=16, sl=16, qsl=16, nct=16, scale=1.0, R=1, T=1, Hq=8,
             Hkv=2, D=64, NB=4, MB=2, mql=1, msl=32, dtype=1, ws=256, wsb=1 << 20, stream=None)
    a.update(kw)
    ptr = lambda x: x
    return lib.paged_attention(a["out"] if "out" in kw else 16, a["q"] if "q" in kw else 16,
                               a["kv"], a["bt"], a["sl"], a["qsl"], a["nct"], a["scale"], a["R"],
                               a["T"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["MB"], a["mql"],
                               a["msl"], a["dtype"], a["ws"], a["wsb"], a["stream"])


def test_attention_rejects_bad_arguments_before_launch():
    import paged_kv_cache_61_amd as pkv
    lib = pkv._lib
    assert _attn(lib, dtype=7) == 3
    assert _attn(lib, Hq=6, Hkv=4) == 2
    assert _attn(lib, Hq=34, Hkv=2) == 2            # group > 16
    assert _attn(lib, D=96) == 2
    assert _attn(lib, R=-1) == 2
    assert _attn(lib, NB=0) == 2
    assert _attn(lib, scale=float("nan")) == 2
    assert _attn(lib, out=None) == 1
    assert _attn(lib, ws=None) == 1
    assert _attn(lib, bt=None) == 1
    assert _attn(lib, kv=24) == 7                   # misaligned
    assert _attn(lib, ws=16 + 256) == 7
    assert _attn(lib, ws=512, wsb=64) == 4          # workspace too small
    assert "workspace" in pkv.last_error_detail()


def test_write_rejects_bad_arguments_before_launch():
    import paged_kv_cache_61_amd as pkv
    lib = pkv._lib
    base = dict(k=16, v=16, sm=16, kv=16, T=4, NB=4, Hkv=2, D=64, dtype=0)

    def call(**kw):
        a = dict(base, **kw)
        return lib.paged_kv_write(a["k"], a["v"], a["sm"], a["kv"], a["T"], a["NB"], a["Hkv"],
                                  a["D"], a["dtype"], None, None)
    assert call(dtype=5) == 3
    assert call(T=-1) == 2
    assert call(D=80) == 2
    assert call(NB=0) == 2
    assert call(kv=None) == 1
    assert call(k=None) == 1
    assert call(k=8) == 7
    assert call(T=0, k=None, v=None, sm=None) == 0  # nothing to do


def test_workspace_size():
    import paged_kv_cache_61_amd as pkv
    small = pkv.paged_attention_workspace_size(4, 4, 8, 64, 1, 64)
    big = pkv.paged_attention_workspace_size(8, 8, 64, 128, 1, 32768)
    assert 0 < small < big
    # 8 rows x 32 partitions (1024 tokens each) x 64 heads x (128 + 2) floats
    # of partials at least
    assert big >= 8 * 32 * 64 * 130 * 4
    assert pkv.paged_attention_workspace_size(-1, 4, 8, 64, 1, 64) == 0


def test_host_metadata_validator():
    import paged_kv_cache_61_amd as pkv
    import workloads
    wl = workloads.build(workloads.small_spec("v", 1, "f32", 4, 2, 64, [(3, 1), (0, 20), (40, 2)]))
    args = lambda **kw: dict(block_table=wl.block_table, seq_lens=wl.seq_lens,
                             query_start_loc=wl.query_start_loc,
                             num_computed_tokens=wl.num_computed_tokens,
                             slot_mapping=wl.slot_mapping, num_tokens=wl.num_tokens,
                             num_blocks=wl.num_blocks, max_query_len=wl.max_query_len,
                             max_seq_len=wl.max_seq_len) | kw
    assert pkv.pkv_validate_metadata_host(**args()) == 0
    bad = wl.seq_lens.copy(); bad[1] += 1
    assert pkv.pkv_validate_metadata_host(**args(seq_lens=bad)) == 6
    bt = wl.block_table.copy(); bt[2, 0] = wl.num_blocks
    assert pkv.pkv_validate_metadata_host(**args(block_table=bt)) == 6
    qsl = wl.query_start_loc.copy(); qsl[1], qsl[2] = qsl[2], qsl[1]
    assert pkv.pkv_validate_metadata_host(**args(query_start_loc=qsl)) == 6
    sm = wl.slot_mapping.copy(); sm[1] = sm[0]
    assert pkv.pkv_validate_metadata_host(**args(slot_mapping=sm)) == 6
    sm = wl.slot_mapping.copy(); sm[0] = -1
    assert pkv.pkv_validate_metadata_host(**args(slot_mapping=sm)) == 0
    sm[0] = -2
    assert pkv.pkv_validate_metadata_host(**args(slot_mapping=sm)) == 6
    assert pkv.pkv_validate_metadata_host(**args(max_seq_len=10)) == 6
    assert pkv.pkv_validate_metadata_host(**args(max_query_len=1)) == 6


def test_noalloc_rejects_steps_beyond_its_scratch():
    import paged_kv_cache_61_amd as pkv
    lib = pkv._lib
    args = lambda R, T, Hq, Hkv, D, mql, msl, dtype=1: (16, 16, 16, 16, 16, 16, 16, 1.0, R, T, Hq, Hkv, D, 64, 4,
                                                        mql, msl, dtype, None, None)
    need = pkv.paged_attention_workspace_size(64, 64, 64, 128, 1, 1 << 20)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    assert lib.paged_attention_noalloc(*args(64, 64, 64, 8, 128, 1, 1 << 20)) == 4   # returns before any HIP call
    assert "static scratch" in pkv.last_error_detail()
    assert lib.paged_attention_noalloc(*args(64, 64, 64, 8, 128, 1, 1 << 20, dtype=9)) == 3
    assert lib.paged_attention_noalloc(*args(64, 64, 6, 4, 128, 1, 4096)) == 2
