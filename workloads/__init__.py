"""Seeded synthetic inputs for attention over a paged KV cache.

This module is shared by the oracle-side tests and the GPU path's tests and
benchmark.  It only *draws* inputs: lengths, a block assignment, the cache pool
contents, the new tokens' K/V and their slots.  It holds none of the attention
arithmetic (no scores, no softmax, no weighted sums).

Layout of the inputs (from "AI Infra入门干货总结：大模型是如何高效推理的",
section "Paged Attention"):

* one layer of the KV cache is ``pool[2, num_blocks, 16, num_kv_heads, head_dim]``
  (K at index 0, V at index 1, 16 tokens per block, token-major inside a block);
* ``block_table[num_reqs, max_blocks_per_req]`` holds physical block ids;
* ``slot_mapping[t] = block * 16 + offset`` places new token ``t``.

Recipe (the same for every workload):

* ``numpy.random.default_rng([seed, stream, chunk])``: stream 0 lengths,
  1 block permutation, 2 q, 3 pool K, 4 pool V, 5 new K, 6 new V.
* Values are N(0,1) float32; bf16 workloads round them to nearest-even bf16 and
  keep the raw 16-bit patterns (``uint16`` arrays).
* Every slot of a block that some request uses gets its own random value.
  Slots that no request may read hold NaN: the tail of each request's last
  block, whole unused blocks, and one extra poison block (the last physical
  block) that every unused ``block_table`` entry points at.  The slots of the
  step's new tokens also hold NaN until ``paged_kv_write`` fills them.
* Physical blocks are handed out by walking a seeded permutation of the pool.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 25  # elements per independently seeded chunk


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits.

    Finite inputs only (the generators never draw NaN or Inf here)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _fill_normal(out_flat: np.ndarray, seed: int, stream: int, bf16: bool) -> None:
    """Fill ``out_flat`` with N(0,1) draws, chunk ``c`` seeded by (seed, stream, c)."""
    n = out_flat.size
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.default_rng([seed, stream, c])
        v = g.standard_normal(hi - lo, dtype=np.float32)
        out_flat[lo:hi] = bf16_bits_from_f32(v) if bf16 else v

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
        return
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))


def normal_array(shape: Sequence[int], seed: int, stream: int, dtype: str) -> np.ndarray:
    """Seeded N(0,1) array: float32, or bf16 bit patterns (uint16)."""
    bf16 = dtype == "bf16"
    out = np.empty(int(np.prod(shape)), dtype=np.uint16 if bf16 else np.float32)
    _fill_normal(out, seed, stream, bf16)
    return out.reshape(shape)


@dataclasses.dataclass(frozen=True)
class Spec:
    """What one synthetic step looks like.

    ``requests(rng)`` returns a list of ``(num_computed_tokens, query_len)``.
    ``pool_blocks``: size of the physical pool without the poison block;
    ``None`` sizes it to exactly the blocks the requests need."""
    name: str
    seed: int
    dtype: str                       # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    requests: Callable[[np.random.Generator], List[Tuple[int, int]]]
    pool_blocks: Optional[int] = None


@dataclasses.dataclass
class Workload:
    spec: Spec
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int                  # physical blocks including the poison block
    max_blocks_per_req: int
    scale: float
    q: np.ndarray                    # [T, Hq, D]
    pool: np.ndarray                 # [2, num_blocks, 16, Hkv, D], before the step's write
    k_new: np.ndarray                # [T, Hkv, D]
    v_new: np.ndarray                # [T, Hkv, D]
    slot_mapping: np.ndarray         # [T] int64
    block_table: np.ndarray          # [R, max_blocks_per_req] int32
    seq_lens: np.ndarray             # [R] int32
    query_start_loc: np.ndarray      # [R+1] int32
    num_computed_tokens: np.ndarray  # [R] int32

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_reqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_reqs else 0


def build(spec: Spec) -> Workload:
    """Draw one workload from ``spec`` (deterministic in ``spec.seed``)."""
    seed = spec.seed
    bf16 = spec.dtype == "bf16"
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    reqs = spec.requests(np.random.default_rng([seed, 0]))
    R = len(reqs)
    nct = np.array([c for c, _ in reqs], dtype=np.int32)
    ql = np.array([q for _, q in reqs], dtype=np.int32)
    L = (nct + ql).astype(np.int32)
    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    T = int(qsl[-1])
    nblk = (L + BLOCK - 1) // BLOCK
    need = int(nblk.sum())
    pool_blocks = need if spec.pool_blocks is None else int(spec.pool_blocks)
    if pool_blocks < need:
        raise ValueError(f"{spec.name}: pool of {pool_blocks} blocks < {need} needed")
    NB = pool_blocks + 1
    poison = pool_blocks
    MB = max(1, int(nblk.max()) if R else 1)

    perm = np.random.default_rng([seed, 1]).permutation(pool_blocks).astype(np.int32)
    bt = np.full((R, MB), poison, dtype=np.int32)
    starts = np.zeros(R + 1, dtype=np.int64)
    starts[1:] = np.cumsum(nblk)
    for r in range(R):
        bt[r, : nblk[r]] = perm[starts[r]: starts[r + 1]]

    # Pool: random everywhere, then NaN where nothing may be read.
    pool = np.empty((2, NB, BLOCK, Hkv, D), dtype=np.uint16 if bf16 else np.float32)
    half = pool.reshape(2, -1)
    _fill_normal(half[0], seed, 3, bf16)
    _fill_normal(half[1], seed, 4, bf16)
    nan = BF16_NAN if bf16 else np.float32(np.nan)
    used = np.zeros(NB, dtype=bool)
    used[perm[:need]] = True
    unused = np.nonzero(~used)[0]
    pool[:, unused] = nan

    def slots_of(r: int, pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        return bt[r, pos // BLOCK], pos % BLOCK

    tail_b, tail_o = [], []
    new_b, new_o = [], []
    slot_mapping = np.empty(T, dtype=np.int64)
    for r in range(R):
        pos_tail = np.arange(int(L[r]), int(nblk[r]) * BLOCK)
        if pos_tail.size:
            b, o = slots_of(r, pos_tail)
            tail_b.append(b), tail_o.append(o)
        pos_new = np.arange(int(nct[r]), int(L[r]))
        if pos_new.size:
            b, o = slots_of(r, pos_new)
            new_b.append(b), new_o.append(o)
            slot_mapping[qsl[r]: qsl[r + 1]] = b.astype(np.int64) * BLOCK + o
    for bs, os_ in ((tail_b, tail_o), (new_b, new_o)):
        if bs:
            b = np.concatenate(bs)
            o = np.concatenate(os_)
            pool[0, b, o] = nan
            pool[1, b, o] = nan

    dt = spec.dtype
    q = normal_array((T, Hq, D), seed, 2, dt)
    k_new = normal_array((T, Hkv, D), seed, 5, dt)
    v_new = normal_array((T, Hkv, D), seed, 6, dt)
    return Workload(spec=spec, dtype=dt, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    num_blocks=NB, max_blocks_per_req=MB, scale=1.0 / math.sqrt(D),
                    q=q, pool=pool, k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
                    block_table=bt, seq_lens=L, query_start_loc=qsl,
                    num_computed_tokens=nct)


# ---------------------------------------------------------------------------
# The five workloads.  Lengths are inclusive integer ranges.

def _decode(lengths: np.ndarray) -> List[Tuple[int, int]]:
    return [(int(x) - 1, 1) for x in lengths]


def _tiny_decode(g):
    return _decode(g.integers(1, 65, size=4))


def _llama7b_decode(g):
    return _decode(g.integers(512, 4097, size=64))


def _lognormal_decode(g):
    x = np.exp(math.log(1024.0) + 0.8 * g.standard_normal(256))
    return _decode(np.clip(np.rint(x), 16, 8192).astype(np.int64))


def _mixed_step(g):
    pre = [(0, 2048), (1024, 2048), (4096, 2048)]
    return pre + _decode(g.integers(256, 2049, size=2048))


def _long_decode(g):
    return _decode(np.full(8, 32768))


BENCH_WORKLOADS = {
    1: Spec("tiny paged decode fp32 (4 seqs, L~U[1,64], 8q/2kv, D=64, pool 64)",
            1, "f32", 8, 2, 64, _tiny_decode, pool_blocks=64),
    2: Spec("Llama-7B-shaped decode bf16 (64 seqs, L~U[512,4096], 32q/32kv, D=128)",
            2, "bf16", 32, 32, 128, _llama7b_decode),
    3: Spec("GQA decode bf16 (256 seqs, L lognormal med 1024, 32q/8kv, D=128)",
            3, "bf16", 32, 8, 128, _lognormal_decode),
    4: Spec("mixed step bf16 (3x2048 prefill on 0/1024/4096 cached + 2048 decodes, 32q/8kv)",
            4, "bf16", 32, 8, 128, _mixed_step),
    5: Spec("long-context split-KV decode bf16 (8 seqs x 32768, 64q/8kv, D=128)",
            5, "bf16", 64, 8, 128, _long_decode),
}


def small_spec(name: str, seed: int, dtype: str, hq: int, hkv: int, d: int,
               reqs: Sequence[Tuple[int, int]], pool_blocks: Optional[int] = None) -> Spec:
    """A fixed-request spec for tests (requests given as (computed, query_len))."""
    fixed = [tuple(map(int, x)) for x in reqs]
    return Spec(name, seed, dtype, hq, hkv, d, lambda g: list(fixed), pool_blocks)


def random_spec(name: str, seed: int, dtype: str, hq: int, hkv: int, d: int,
                num_reqs: int, max_ctx: int, max_ql: int, decode_frac: float = 0.5) -> Spec:
    """A seeded ragged mixed batch for tests: some decodes, some prefill chunks."""
    def gen(g):
        out = []
        for _ in range(num_reqs):
            if g.random() < decode_frac:
                out.append((int(g.integers(0, max_ctx)), 1))
            else:
                out.append((int(g.integers(0, max_ctx)), int(g.integers(1, max_ql + 1))))
        return out
    return Spec(name, seed, dtype, hq, hkv, d, gen)
