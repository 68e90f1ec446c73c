// Step planning on the device: from query_start_loc, seq_lens and
// num_computed_tokens, check each request and turn the step into work lists.
//
// Continuous batching ("AI Infra入门干货总结：大模型是如何高效推理的",
// section "连续批处理") schedules, per request, the tokens between
// num_computed_tokens and num_tokens, with no separate prefill and decode
// phases; one step therefore mixes single-token decodes and multi-token
// prefill chunks.  This kernel sorts them:
//   query_len == 1  -> decode row; split into 1024-token partitions when the
//                      row is longer than one partition (split-KV), plus one
//                      reduce item that merges the partitions;
//   query_len  > 1  -> prefill tiles for the MFMA kernel (bf16), or one row
//                      item per query row (fp32);
//   query_len == 0  -> nothing.
// Row items are listed longest first (full partitions and whole rows, then
// the partial last partitions) for the row kernel's persistent workers.
// The partition count depends only on the row's own length, so a request's
// result is the same whatever else is in the batch.
//
// One workgroup of 1024 threads walks the requests 1024 at a time and places
// each request's items with a block-wide exclusive scan.  No host sync is
// needed: the later kernels read the counts from the workspace header.
#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;

struct Counts {
  int rows, prefill, reduce, slots, tail;
};

// Exclusive scan of the five counters over the workgroup; returns the prefix
// and writes the workgroup total to `total`.
constexpr int kNC = 5;
__device__ Counts block_exclusive_scan(Counts c, Counts* total) {
  __shared__ int wave_tot[kPlanWaves][kNC];
  __shared__ int wave_off[kPlanWaves][kNC];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  int v[kNC] = {c.rows, c.prefill, c.reduce, c.slots, c.tail};
  int inc[kNC];
#pragma unroll
  for (int j = 0; j < kNC; ++j) {
    int x = v[j];
    for (int off = 1; off < kWave; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    inc[j] = x;
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int j = 0; j < kNC; ++j) wave_tot[w][j] = inc[j];
  }
  __syncthreads();
  if (threadIdx.x < kNC) {
    int run = 0;
    for (int i = 0; i < kPlanWaves; ++i) {
      wave_off[i][threadIdx.x] = run;
      run += wave_tot[i][threadIdx.x];
    }
    wave_tot[0][threadIdx.x] = run;  // reuse row 0 for the totals
  }
  __syncthreads();
  Counts ex{inc[0] - v[0] + wave_off[w][0], inc[1] - v[1] + wave_off[w][1],
            inc[2] - v[2] + wave_off[w][2], inc[3] - v[3] + wave_off[w][3],
            inc[4] - v[4] + wave_off[w][4]};
  *total = Counts{wave_tot[0][0], wave_tot[0][1], wave_tot[0][2], wave_tot[0][3], wave_tot[0][4]};
  __syncthreads();
  return ex;
}

// Buckets of the counting sorts that list work longest first.
constexpr int kPfBuckets = 4096;          // prefill tiles by KV tiles to read (clamped)
static_assert(kPfBuckets % 1024 == 0, "buckets split evenly over the plan threads");
constexpr int kTailBuckets = kSplitBlocks; // partial partitions by block count

struct ReqInfo {
  int kind;  // 0 none, 1 decode row, 2 prefill tiles, 3 rows per query, 4 NaN rows
  int qs, ql, L, c, nparts, err;
};

__device__ ReqInfo classify(const PlanParams& a, int r) {
  ReqInfo q{0, 0, 0, 0, 0, 1, 0};
  if (r >= a.num_reqs) return q;
  q.qs = a.qsl[r];
  const int qe = a.qsl[r + 1];
  q.ql = qe - q.qs;
  q.L = a.seq_lens[r];
  q.c = a.nct[r];
  const bool qsl_ok = q.qs >= 0 && q.ql >= 0 && (int64_t)qe <= a.num_tokens && (r > 0 || q.qs == 0);
  if (!qsl_ok) {
    q.err |= PKV_DEVERR_QSL;
  } else if (q.c < 0 || q.L != q.c + q.ql) {
    q.err |= PKV_DEVERR_SEQ_LEN;
    q.kind = 4;
  } else if (q.ql > a.max_query_len || q.L > a.max_seq_len || q.L > a.max_blocks_per_req * kBlock) {
    q.err |= PKV_DEVERR_LIMITS;
    q.kind = 4;
  } else if (q.ql == 1) {
    q.kind = 1;
    q.nparts = a.split_decode ? (q.L + kSplitTokens - 1) / kSplitTokens : 1;
  } else if (q.ql > 1) {
    q.kind = a.mfma_prefill ? 2 : 3;
  }
  if (q.kind == 4 && q.ql == 0) q.kind = 0;
  return q;
}

// KV tiles (of 64 keys) a prefill tile starting at query row0 with `rows`
// rows reads: its bucket in the longest-first order.
__device__ int pf_bucket(const ReqInfo& q, int row0, int rows) {
  const int kv_end = q.c + row0 + rows;
  return min((kv_end + 63) / 64, kPfBuckets - 1);
}

// Wave-wide maximum of an int (all 64 lanes active): rotations inside rows
// of 16 lanes (DPP), then the v_permlane16/32 swaps; VALU only.
template <int CTRL>
PKV_DEV int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
PKV_DEV int wave_max_i(int x) {
  x = max(x, dpp_i<0x121>(x));  // row_ror:1
  x = max(x, dpp_i<0x122>(x));  // row_ror:2
  x = max(x, dpp_i<0x124>(x));  // row_ror:4
  x = max(x, dpp_i<0x128>(x));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = max((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return max((int)r[0], (int)r[1]);
}

// Static assignment of the prefill items to the W workgroups of each kv head
// (every head has the same item list): first fit decreasing on a cost of
// (10 * tiles + 50) per item (KV tiles to read plus the item's fixed
// overhead of about five tile periods, in tenths of a tile).  Items arrive
// longest first; each goes to the lowest slot it still fits in under the
// capacity ceil(total / W) + 5, or else to the emptiest slot, ties to the
// lowest.  On this list first fit packs as tightly as best fit and needs one
// ballot per item instead of a wave-wide maximum.  An item costing more than
// half the capacity fits in no slot that already holds one (those hold items
// at least as long), so the first such items, up to W, take slots 0, 1, ...
// directly; the rest are placed one by one.  Lane s of the calling wave holds
// slot s's load and item count (loads stay below 2^24: at most 256 items of
// at most 4095 tiles).  Writes slot_of[i] and the item's rank inside its
// slot, then the slot offsets (exclusive sums of the counts).
PKV_DEV int item_cost(int tiles) { return 10 * tiles + 50; }

PKV_DEV void assign_first_fit(const int* tiles, int n, int W, int* slot_of, int* rank_of, int* slot_start) {
  const int lane = threadIdx.x & (kWave - 1);
  int total = 0, big = 0;
  for (int i = lane; i < n; i += kWave) total += item_cost(tiles[i]);
  for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
  const int cap = (total + W - 1) / W + 5;
  for (int i = lane; i < n; i += kWave) big += 2 * item_cost(tiles[i]) > cap ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) big += __shfl_xor(big, off);
  const int p = min(big, W);                        // items placed directly: item i in slot i
  const bool live = lane < W;
  int load = lane < p ? item_cost(tiles[lane]) : 0;
  int cnt = lane < p ? 1 : 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int tl = i0 + lane < n ? tiles[i0 + lane] : 0;
    int slot = i0 + lane < p ? i0 + lane : 0, rank = 0;   // for item i0 + lane
    for (int j = max(p - i0, 0); j < kWave && i0 + j < n; ++j) {
      const int c = item_cost(__builtin_amdgcn_readlane(tl, j));
      const uint64_t fits = __ballot(live && load + c <= cap);
      int win;
      if (fits) {
        win = __builtin_ctzll(fits);
      } else {   // no slot has room: the emptiest one
        const int m = wave_max_i(live ? ((0xffffff - load) << 6) | (63 - lane) : -1);
        win = 63 - (__builtin_amdgcn_readfirstlane(m) & 63);
      }
      const int r = __builtin_amdgcn_readlane(cnt, win);
      const bool mine = lane == win;
      load += mine ? c : 0;
      cnt += mine ? 1 : 0;
      slot = lane == j ? win : slot;
      rank = lane == j ? r : rank;
    }
    if (i0 + lane < n) {
      slot_of[i0 + lane] = slot;
      rank_of[i0 + lane] = rank;
    }
  }
  // exclusive sums of the counts (W <= 64 lanes)
  __shared__ int cnt_lds[kPfMaxSlots];
  cnt_lds[lane] = cnt;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int st = 0;
  for (int j = 0; j < lane; ++j) st += cnt_lds[j];
  if (lane < W) slot_start[lane] = st;
  if (lane == 0) slot_start[W] = n;   // W may be 64: no lane W
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams a) {
  __shared__ int err_acc;
  __shared__ int pf_tiles[kPfMaxStatic], pf_slot_of[kPfMaxStatic], pf_rank[kPfMaxStatic];
  __shared__ int pf_start[kPfMaxSlots + 1];
  __shared__ int pf_off[kPfBuckets];
  __shared__ int tail_off[kTailBuckets];
  for (int i = threadIdx.x; i < kPfBuckets; i += kPlanThreads) pf_off[i] = 0;
  if (threadIdx.x < kTailBuckets) tail_off[threadIdx.x] = 0;
  if (threadIdx.x == 0) err_acc = 0;
  __syncthreads();

  // Pass 1: check requests, place decode rows (full partitions) and reduce
  // items, count everything, and histogram the items that are sorted.
  Counts base{0, 0, 0, 0, 0};
  ReqInfo first{};  // this thread's request of the first pass, reused by pass 2
  for (int r0 = 0; r0 < a.num_reqs; r0 += kPlanThreads) {
    const int r = r0 + threadIdx.x;
    const ReqInfo q = classify(a, r);
    if (r0 == 0) first = q;
    int err = q.err;
    const bool partial_last = q.kind == 1 && q.L % kSplitTokens != 0;
    Counts mine{0, 0, 0, 0, 0};
    if (q.kind == 1) {
      mine.rows = q.nparts - (partial_last ? 1 : 0);
      mine.tail = partial_last ? 1 : 0;
      if (q.nparts > 1) {
        mine.reduce = 1;
        mine.slots = q.nparts;
      }
    } else if (q.kind == 2) {
      mine.prefill = (q.ql + a.prefill_tile_rows - 1) / a.prefill_tile_rows;
    } else if (q.kind == 3 || q.kind == 4) {
      mine.rows = q.ql;
    }
    Counts tot;
    Counts ex = block_exclusive_scan(mine, &tot);
    ex.rows += base.rows;
    ex.reduce += base.reduce;
    ex.slots += base.slots;
    const bool fits = ex.rows + mine.rows <= a.cap_row_items &&
                      base.tail + tot.tail <= a.cap_row_items &&
                      base.prefill + tot.prefill <= a.cap_prefill_items &&
                      ex.reduce + mine.reduce <= a.cap_reduce && ex.slots + mine.slots <= a.cap_slots;
    if (!fits) {
      err |= PKV_DEVERR_CAPACITY;
    } else if (q.kind == 1) {
      const int nfull = q.nparts - (partial_last ? 1 : 0);
      for (int p = 0; p < nfull; ++p)
        a.row_items[ex.rows + p] =
            make_int4(q.qs, r, q.nparts == 1 ? kWholeRow : p, q.nparts == 1 ? -1 : ex.slots);
      if (partial_last) atomicAdd(&tail_off[(q.L % kSplitTokens + kBlock - 1) / kBlock - 1], 1);
      if (q.nparts > 1) a.reduce_items[ex.reduce] = make_int4(q.qs, r, q.nparts, ex.slots);
    } else if (q.kind == 2) {
      for (int row0 = 0; row0 < q.ql; row0 += a.prefill_tile_rows)
        atomicAdd(&pf_off[pf_bucket(q, row0, min(a.prefill_tile_rows, q.ql - row0))], 1);
    } else if (q.kind == 3 || q.kind == 4) {
      const int z = q.kind == 3 ? kWholeRow : kNanRow;
      for (int i = 0; i < q.ql; ++i) a.row_items[ex.rows + i] = make_int4(q.qs + i, r, z, -1);
    }
    if (err) atomicOr(&err_acc, err);
    base.rows += tot.rows;
    base.prefill += tot.prefill;
    base.reduce += tot.reduce;
    base.slots += tot.slots;
    base.tail += tot.tail;
  }
  __syncthreads();
  const bool over = base.rows > a.cap_row_items || base.tail > a.cap_row_items ||
                    base.prefill > a.cap_prefill_items || base.reduce > a.cap_reduce ||
                    base.slots > a.cap_slots;
  // Bucket offsets, longest bucket first: thread t owns the 4 buckets at
  // descending positions 4t .. 4t+3 of the prefill list; thread 0 also does
  // the 32 tail buckets.  (Skipped, like pass 2, when nothing is sorted:
  // base is the same in every thread.)
  const bool sorted_work = base.prefill > 0 || base.tail > 0;
  if (sorted_work) {
    constexpr int kPer = kPfBuckets / kPlanThreads;
    int n[kPer], local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      n[i] = pf_off[kPfBuckets - 1 - (kPer * threadIdx.x + i)];
      local += n[i];
    }
    Counts tot;
    int run = block_exclusive_scan(Counts{local, 0, 0, 0, 0}, &tot).rows;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      pf_off[kPfBuckets - 1 - (kPer * threadIdx.x + i)] = run;
      run += n[i];
    }
    if (threadIdx.x == 0) {
      int trun = 0;
      for (int b = kTailBuckets - 1; b >= 0; --b) {
        const int m = tail_off[b];
        tail_off[b] = trun;
        trun += m;
      }
    }
  }
  __syncthreads();

  // Pass 2: scatter the sorted items (order inside a bucket is irrelevant:
  // an item's result does not depend on which worker computes it).
  if (!over && sorted_work) {
    int slot_base = 0;  // the split rows' partial slots, recomputed as in pass 1
    for (int r0 = 0; r0 < a.num_reqs; r0 += kPlanThreads) {
      const int r = r0 + threadIdx.x;
      const ReqInfo q = r0 == 0 ? first : classify(a, r);
      Counts mine{0, 0, 0, 0, 0};
      if (q.kind == 1 && q.nparts > 1) mine.slots = q.nparts;
      Counts tot;
      const int slot0 = block_exclusive_scan(mine, &tot).slots + slot_base;
      slot_base += tot.slots;
      if (q.kind == 1 && q.L % kSplitTokens != 0) {
        const int nb = (q.L % kSplitTokens + kBlock - 1) / kBlock;
        const int pos = atomicAdd(&tail_off[nb - 1], 1);
        a.row_items_tail[pos] = q.nparts == 1 ? make_int4(q.qs, r, kWholeRow, -1)
                                              : make_int4(q.qs, r, q.nparts - 1, slot0);
      } else if (q.kind == 2) {
        for (int row0 = 0; row0 < q.ql; row0 += a.prefill_tile_rows) {
          const int rows = min(a.prefill_tile_rows, q.ql - row0);
          const int tiles = pf_bucket(q, row0, rows);
          const int pos = atomicAdd(&pf_off[tiles], 1);
          a.prefill_items[pos] = make_int4(r, q.qs + row0, rows, q.c - q.qs);
          if (pos < kPfMaxStatic) pf_tiles[pos] = tiles;
        }
      }
    }
  }
  __syncthreads();
  // Static prefill assignment when it is small enough to build here (one
  // wave); otherwise the prefill kernel takes items from per-head queues.
  const int npf = base.prefill;
  const bool pf_static = !over && npf > 0 && npf <= kPfMaxStatic && a.prefill_slots > 0 &&
                         a.prefill_slots <= kPfMaxSlots;
  if (pf_static && threadIdx.x < kWave) assign_first_fit(pf_tiles, npf, a.prefill_slots, pf_slot_of, pf_rank, pf_start);
  __syncthreads();
  if (pf_static) {
    for (int i = threadIdx.x; i < npf; i += blockDim.x) a.pf_order[pf_start[pf_slot_of[i]] + pf_rank[i]] = i;
    for (int i = threadIdx.x; i <= a.prefill_slots; i += blockDim.x) a.pf_slot_start[i] = pf_start[i];
  }
  for (int i = threadIdx.x; i < kMaxKvHeads; i += blockDim.x) a.hdr[kHdrPrefillQueue + i] = 0;
  if (threadIdx.x == 0) {
    // On overflow nothing past the capacity was written; run no work at all.
    a.hdr[kHdrError] = err_acc | (over ? PKV_DEVERR_CAPACITY : 0);
    a.hdr[kHdrRowItems] = over ? 0 : base.rows + base.tail;
    a.hdr[kHdrRowHead] = over ? 0 : base.rows;
    a.hdr[kHdrPrefillItems] = over ? 0 : base.prefill;
    a.hdr[kHdrPrefillStatic] = pf_static ? 1 : 0;
    a.hdr[kHdrReduceItems] = over ? 0 : base.reduce;
    a.hdr[kHdrSlots] = over ? 0 : base.slots;
  }
}

}  // namespace

int launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
