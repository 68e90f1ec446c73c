"""Reference block manager and step scheduler (plain Python).

TEST INFRASTRUCTURE.  Only the tests may import or run this module; the
product library never does, and this module shares no code with the C++
block manager it checks (``paged_kv_cache_61_amd/csrc/block_manager.cpp``).

What it models, and where each rule comes from:

* The cache is a pool of fixed-size blocks of 16 tokens, allocated up front;
  each sequence has a block table listing its blocks, and when a sequence's
  last block is full the next free block is taken (lpnh.cn/news/2436702,
  section 2.2, "Block 管理器").  A request's pages are allocated when it
  arrives, appended to as it grows and returned to the pool when it finishes
  ("大模型推理部署：从单卡到集群的工程化落地路径", section 2.2, the
  allocate / append / free sequence).
* Sequences that start with the same prompt share the prefix blocks, and a
  block is copied only when the sequences diverge inside it (copy-on-write;
  lpnh.cn/news/2436702, section 2.2).  Tokens found in shared cached blocks
  count as computed ("AI Infra入门干货总结", section "连续批处理":
  num_computed_tokens includes prefix-cache hits).
* The scheduler has no prefill or decode phase: each step it schedules, per
  request, the tokens between ``num_computed_tokens`` and ``num_tokens``,
  under four limits: the number of requests in a step, the step's token
  budget, the model's maximum length, and the free blocks (same page, same
  section, "4个硬性约束").

Readings where the pages are silent:

* Requests are served first come, first served; a request that cannot get a
  block this step is skipped (it waits; no preemption), and later requests may
  still be scheduled.
* A request gets as many of its pending tokens as the budget, the maximum
  length and the free blocks allow (a partial chunk is a chunked prefill).
* Free blocks are handed out in first-in, first-out order: initially 0, 1, 2,
  ...; a freed block goes to the back of the queue (a finished request frees
  its blocks in table order).
* A shared block is copied before a step writes into it: that only happens
  to a partially filled last block, since full blocks are never written
  again.  The copy takes a free block first, before any new block of the
  request.
* Unused block-table entries are -1.
"""
from __future__ import annotations

from collections import OrderedDict, deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class _Req:
    num_tokens: int
    num_computed: int
    blocks: List[int] = field(default_factory=list)


@dataclass
class Step:
    req_ids: np.ndarray            # int64 [R]
    query_start_loc: np.ndarray    # int32 [R + 1]
    seq_lens: np.ndarray           # int32 [R]
    num_computed_tokens: np.ndarray  # int32 [R]
    block_table: np.ndarray        # int32 [R, max_blocks_per_req], -1 = unused
    slot_mapping: np.ndarray       # int64 [T]
    copies: np.ndarray             # int32 [C, 2]: (source block, destination block)

    @property
    def num_reqs(self) -> int:
        return int(self.req_ids.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])


class BlockManager:
    def __init__(self, num_blocks: int, max_blocks_per_req: int):
        self.num_blocks = num_blocks
        self.max_blocks_per_req = max_blocks_per_req
        self.free = deque(range(num_blocks))
        self.ref = [0] * num_blocks
        self.reqs: "OrderedDict[int, _Req]" = OrderedDict()
        self.pending: Optional[List[Tuple[int, int]]] = None

    # -- request lifecycle ---------------------------------------------------

    def add_request(self, req_id: int, num_prompt_tokens: int,
                    prefix_from: Optional[int] = None, prefix_tokens: int = 0) -> None:
        """A new request of ``num_prompt_tokens``.  With ``prefix_from``, the
        first ``prefix_tokens // 16`` blocks of that request (tokens it has
        already computed) are shared and count as computed."""
        assert self.pending is None and req_id not in self.reqs and num_prompt_tokens >= 1
        r = _Req(num_prompt_tokens, 0)
        if prefix_from is not None:
            src = self.reqs[prefix_from]
            nshare = min(prefix_tokens, src.num_computed, num_prompt_tokens - 1) // BLOCK_SIZE
            for b in src.blocks[:nshare]:
                self.ref[b] += 1
                r.blocks.append(b)
            r.num_computed = nshare * BLOCK_SIZE
        self.reqs[req_id] = r

    def fork(self, parent_id: int, child_id: int) -> None:
        """The child continues from the parent's state and shares all of its
        blocks (copy-on-write)."""
        assert self.pending is None and child_id not in self.reqs
        p = self.reqs[parent_id]
        for b in p.blocks:
            self.ref[b] += 1
        self.reqs[child_id] = _Req(p.num_tokens, p.num_computed, list(p.blocks))

    def append_tokens(self, req_id: int, n: int = 1) -> None:
        assert self.pending is None and n >= 0
        self.reqs[req_id].num_tokens += n

    def finish(self, req_id: int) -> None:
        assert self.pending is None
        r = self.reqs.pop(req_id)
        for b in r.blocks:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- one step --------------------------------------------------------------

    def schedule(self, max_num_seqs: int, token_budget: int, max_model_len: int) -> Step:
        assert self.pending is None
        budget = token_budget
        picked = []   # (req_id, computed, n, blocks snapshot)
        copies = []
        for rid, r in self.reqs.items():
            if len(picked) == max_num_seqs or budget == 0:
                break
            want = r.num_tokens - r.num_computed
            limit = min(max_model_len, self.max_blocks_per_req * BLOCK_SIZE)
            n = min(want, budget, limit - r.num_computed)
            if n <= 0:
                continue
            cow = r.num_computed % BLOCK_SIZE != 0 and self.ref[r.blocks[-1]] > 1
            avail = len(self.free) - (1 if cow else 0)
            if avail < 0:
                continue
            need = _cdiv(r.num_computed + n, BLOCK_SIZE) - len(r.blocks)
            if need > avail:
                n = (len(r.blocks) + avail) * BLOCK_SIZE - r.num_computed
                need = avail
            if n <= 0:
                continue
            if cow:
                old = r.blocks[-1]
                new = self.free.popleft()
                self.ref[old] -= 1
                self.ref[new] = 1
                r.blocks[-1] = new
                copies.append((old, new))
            for _ in range(max(need, 0)):
                b = self.free.popleft()
                self.ref[b] = 1
                r.blocks.append(b)
            picked.append((rid, r.num_computed, n, list(r.blocks)))
            budget -= n
        R = len(picked)
        qsl = np.zeros(R + 1, np.int32)
        bt = np.full((R, self.max_blocks_per_req), -1, np.int32)
        slots = []
        for i, (rid, c, n, blocks) in enumerate(picked):
            qsl[i + 1] = qsl[i] + n
            bt[i, :len(blocks)] = blocks
            for pos in range(c, c + n):
                slots.append(blocks[pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE)
        self.pending = [(rid, n) for rid, c, n, _ in picked]
        return Step(
            req_ids=np.array([p[0] for p in picked], np.int64),
            query_start_loc=qsl,
            seq_lens=np.array([p[1] + p[2] for p in picked], np.int32),
            num_computed_tokens=np.array([p[1] for p in picked], np.int32),
            block_table=bt,
            slot_mapping=np.array(slots, np.int64),
            copies=np.array(copies, np.int32).reshape(-1, 2),
        )

    def commit(self) -> None:
        """The step ran: its scheduled tokens are now in the cache."""
        assert self.pending is not None
        for rid, n in self.pending:
            self.reqs[rid].num_computed += n
        self.pending = None

    # -- inspection ------------------------------------------------------------

    def num_free_blocks(self) -> int:
        return len(self.free)

    def request_state(self, req_id: int) -> Tuple[int, int, List[int]]:
        r = self.reqs[req_id]
        return r.num_tokens, r.num_computed, list(r.blocks)
