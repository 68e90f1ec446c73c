// Host block manager and step scheduler: builds one continuous-batching
// step's metadata (block_table, slot_mapping, seq_lens, query_start_loc,
// num_computed_tokens) for paged_kv_write / paged_attention.
//
// What it implements:
//  * the cache is a pool of 16-token blocks allocated up front; each request
//    has a block table, and when its last block is full the next free block
//    is taken (lpnh.cn/news/2436702, section 2.2, the block manager); blocks
//    are allocated as a request arrives and grows and returned when it
//    finishes ("大模型推理部署：从单卡到集群的工程化落地路径", section 2.2);
//  * requests that share a prompt prefix share its blocks, and a shared block
//    is copied only when a request writes into it (copy-on-write, same page
//    of lpnh.cn, section 2.2); tokens found in shared blocks count as
//    computed ("AI Infra入门干货总结", section "连续批处理");
//  * each step schedules, per request, the tokens between num_computed_tokens
//    and num_tokens, with no prefill / decode distinction, under four limits:
//    requests per step, the step's token budget, the maximum model length
//    and the free blocks (same page and section).
// Where the pages are silent: requests are served first come, first served;
// a request that cannot get a block waits (no preemption) while later ones
// may still run; a request gets as many pending tokens as the limits allow
// (a partial chunk is a chunked prefill); free blocks are handed out first
// in, first out (initially 0, 1, 2, ...; freed blocks join the back, in
// table order); a copy-on-write takes its free block before the request's
// new blocks; unused block-table entries are -1.
//
// Host code only: no HIP call, no device memory.  The copies a step needs
// are returned as (source, destination) pairs for paged_kv_copy_blocks.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "paged_kv.h"
#include "pkv_internal.h"

namespace {

constexpr int32_t kBs = PKV_BLOCK_SIZE;

struct Req {
  int32_t num_tokens = 0;
  int32_t num_computed = 0;
  std::vector<int32_t> blocks;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t max_blocks_per_req = 0;
  std::deque<int32_t> free_q;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Req> reqs;
  std::vector<int64_t> order;                          // arrival order
  bool pending = false;
  std::vector<std::pair<int64_t, int32_t>> scheduled;  // (request, tokens) of the pending step

  void release(Req& r) {
    for (int32_t b : r.blocks)
      if (--ref[b] == 0) free_q.push_back(b);
    r.blocks.clear();
  }
};

extern "C" {

int pkv_bm_create(int32_t num_blocks, int32_t max_blocks_per_req, pkv_block_manager** out) {
  if (!out) return pkv::fail(PKV_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || max_blocks_per_req <= 0)
    return pkv::fail(PKV_ERR_DIMS, "num_blocks %lld, max_blocks_per_req %lld", num_blocks, max_blocks_per_req);
  auto* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return pkv::fail(PKV_ERR_DIMS, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->max_blocks_per_req = max_blocks_per_req;
  bm->ref.assign((size_t)num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) bm->free_q.push_back(b);
  *out = bm;
  return pkv::ok();
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_request_with_prefix(pkv_block_manager* bm, int64_t req_id, int32_t num_prompt_tokens,
                                   int64_t prefix_from, int32_t prefix_tokens) {
  if (!bm) return pkv::fail(PKV_ERR_NULL, "block manager is NULL");
  if (bm->pending) return pkv::fail(PKV_ERR_METADATA, "a scheduled step is not committed");
  if (num_prompt_tokens < 1) return pkv::fail(PKV_ERR_DIMS, "num_prompt_tokens %lld", num_prompt_tokens);
  if (bm->reqs.count(req_id)) return pkv::fail(PKV_ERR_METADATA, "request %lld exists", (long long)req_id);
  Req r;
  r.num_tokens = num_prompt_tokens;
  if (prefix_tokens > 0) {
    auto it = bm->reqs.find(prefix_from);
    if (it == bm->reqs.end())
      return pkv::fail(PKV_ERR_METADATA, "prefix request %lld unknown", (long long)prefix_from);
    const Req& src = it->second;
    // at least one prompt token is left to compute
    const int32_t nshare = std::min({prefix_tokens, src.num_computed, num_prompt_tokens - 1}) / kBs;
    for (int32_t i = 0; i < nshare; ++i) {
      const int32_t b = src.blocks[(size_t)i];
      ++bm->ref[b];
      r.blocks.push_back(b);
    }
    r.num_computed = nshare * kBs;
  }
  bm->reqs.emplace(req_id, std::move(r));
  bm->order.push_back(req_id);
  return pkv::ok();
}

int pkv_bm_add_request(pkv_block_manager* bm, int64_t req_id, int32_t num_prompt_tokens) {
  return pkv_bm_add_request_with_prefix(bm, req_id, num_prompt_tokens, 0, 0);
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return pkv::fail(PKV_ERR_NULL, "block manager is NULL");
  if (bm->pending) return pkv::fail(PKV_ERR_METADATA, "a scheduled step is not committed");
  auto it = bm->reqs.find(parent_id);
  if (it == bm->reqs.end()) return pkv::fail(PKV_ERR_METADATA, "request %lld unknown", (long long)parent_id);
  if (bm->reqs.count(child_id)) return pkv::fail(PKV_ERR_METADATA, "request %lld exists", (long long)child_id);
  Req c = it->second;
  for (int32_t b : c.blocks) ++bm->ref[b];
  bm->reqs.emplace(child_id, std::move(c));
  bm->order.push_back(child_id);
  return pkv::ok();
}

int pkv_bm_append_tokens(pkv_block_manager* bm, int64_t req_id, int32_t n) {
  if (!bm) return pkv::fail(PKV_ERR_NULL, "block manager is NULL");
  if (bm->pending) return pkv::fail(PKV_ERR_METADATA, "a scheduled step is not committed");
  if (n < 0) return pkv::fail(PKV_ERR_DIMS, "n %lld", n);
  auto it = bm->reqs.find(req_id);
  if (it == bm->reqs.end()) return pkv::fail(PKV_ERR_METADATA, "request %lld unknown", (long long)req_id);
  if ((int64_t)it->second.num_tokens + n > INT32_MAX) return pkv::fail(PKV_ERR_DIMS, "too many tokens");
  it->second.num_tokens += n;
  return pkv::ok();
}

int pkv_bm_finish(pkv_block_manager* bm, int64_t req_id) {
  if (!bm) return pkv::fail(PKV_ERR_NULL, "block manager is NULL");
  if (bm->pending) return pkv::fail(PKV_ERR_METADATA, "a scheduled step is not committed");
  auto it = bm->reqs.find(req_id);
  if (it == bm->reqs.end()) return pkv::fail(PKV_ERR_METADATA, "request %lld unknown", (long long)req_id);
  bm->release(it->second);
  bm->reqs.erase(it);
  bm->order.erase(std::find(bm->order.begin(), bm->order.end(), req_id));
  return pkv::ok();
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? (int32_t)bm->free_q.size() : -1; }

int pkv_bm_request_state(const pkv_block_manager* bm, int64_t req_id, int32_t* num_tokens,
                         int32_t* num_computed, int32_t* blocks, int32_t max_blocks, int32_t* num_blocks) {
  if (!bm || !num_tokens || !num_computed || !num_blocks) return pkv::fail(PKV_ERR_NULL, "NULL argument");
  auto it = bm->reqs.find(req_id);
  if (it == bm->reqs.end()) return pkv::fail(PKV_ERR_METADATA, "request %lld unknown", (long long)req_id);
  const Req& r = it->second;
  *num_tokens = r.num_tokens;
  *num_computed = r.num_computed;
  *num_blocks = (int32_t)r.blocks.size();
  if (blocks)
    for (int32_t i = 0; i < std::min<int32_t>(max_blocks, *num_blocks); ++i) blocks[i] = r.blocks[(size_t)i];
  return pkv::ok();
}

int pkv_bm_schedule(pkv_block_manager* bm, pkv_step* st) {
  if (!bm || !st) return pkv::fail(PKV_ERR_NULL, "NULL argument");
  if (bm->pending) return pkv::fail(PKV_ERR_METADATA, "the previous step is not committed");
  if (st->max_num_seqs <= 0 || st->token_budget <= 0 || st->max_model_len <= 0)
    return pkv::fail(PKV_ERR_DIMS, "max_num_seqs %lld, token_budget %lld, max_model_len %lld", st->max_num_seqs,
                     st->token_budget, st->max_model_len);
  if (!st->req_ids || !st->query_start_loc || !st->seq_lens || !st->num_computed_tokens || !st->block_table ||
      !st->slot_mapping || !st->copies)
    return pkv::fail(PKV_ERR_NULL, "a step output array is NULL");
  const int32_t limit = std::min<int64_t>(st->max_model_len, (int64_t)bm->max_blocks_per_req * kBs);
  const size_t mb = (size_t)bm->max_blocks_per_req;
  int32_t budget = st->token_budget;
  int32_t R = 0, T = 0, C = 0, max_ql = 0, max_sl = 0;
  bm->scheduled.clear();
  st->query_start_loc[0] = 0;
  for (int64_t rid : bm->order) {
    if (R == st->max_num_seqs || budget == 0) break;
    Req& r = bm->reqs[rid];
    int64_t n = std::min<int64_t>({(int64_t)r.num_tokens - r.num_computed, budget, limit - r.num_computed});
    if (n <= 0) continue;
    const bool cow = r.num_computed % kBs != 0 && bm->ref[r.blocks.back()] > 1;
    const int64_t avail = (int64_t)bm->free_q.size() - (cow ? 1 : 0);
    if (avail < 0) continue;
    int64_t need = cdiv(r.num_computed + n, kBs) - (int64_t)r.blocks.size();
    if (need > avail) {
      n = ((int64_t)r.blocks.size() + avail) * kBs - r.num_computed;
      need = avail;
    }
    if (n <= 0) continue;
    if (cow) {
      const int32_t old = r.blocks.back();
      const int32_t nb = bm->free_q.front();
      bm->free_q.pop_front();
      --bm->ref[old];
      bm->ref[nb] = 1;
      r.blocks.back() = nb;
      st->copies[2 * C] = old;
      st->copies[2 * C + 1] = nb;
      ++C;
    }
    for (int64_t i = 0; i < need; ++i) {
      const int32_t b = bm->free_q.front();
      bm->free_q.pop_front();
      bm->ref[b] = 1;
      r.blocks.push_back(b);
    }
    st->req_ids[R] = rid;
    st->num_computed_tokens[R] = r.num_computed;
    st->seq_lens[R] = r.num_computed + (int32_t)n;
    st->query_start_loc[R + 1] = T + (int32_t)n;
    int32_t* row = st->block_table + (size_t)R * mb;
    std::fill(row, row + mb, -1);
    std::copy(r.blocks.begin(), r.blocks.end(), row);
    for (int32_t pos = r.num_computed; pos < r.num_computed + n; ++pos)
      st->slot_mapping[T++] = (int64_t)r.blocks[(size_t)(pos / kBs)] * kBs + pos % kBs;
    max_ql = std::max<int32_t>(max_ql, (int32_t)n);
    max_sl = std::max<int32_t>(max_sl, r.num_computed + (int32_t)n);
    bm->scheduled.emplace_back(rid, (int32_t)n);
    budget -= (int32_t)n;
    ++R;
  }
  st->num_reqs = R;
  st->num_tokens = T;
  st->num_copies = C;
  st->max_query_len = max_ql;
  st->max_seq_len = max_sl;
  bm->pending = true;
  return pkv::ok();
}

int pkv_bm_commit(pkv_block_manager* bm) {
  if (!bm) return pkv::fail(PKV_ERR_NULL, "block manager is NULL");
  if (!bm->pending) return pkv::fail(PKV_ERR_METADATA, "no scheduled step");
  for (const auto& s : bm->scheduled) bm->reqs[s.first].num_computed += s.second;
  bm->scheduled.clear();
  bm->pending = false;
  return pkv::ok();
}

}  // extern "C"
