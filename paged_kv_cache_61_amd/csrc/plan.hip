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
// One workgroup of 1024 threads.  Requests are taken 4096 at a time; thread t
// owns a contiguous run of up to 4 of them, loads all their metadata at once
// and keeps it in registers, so a step of up to 4096 requests costs one
// round trip to memory and one block-wide scan (DPP inside each wave, one
// barrier across waves) to place every request's items in request order.
// The longest-first lists are counting sorts: a histogram in LDS, a scan of
// the buckets, then a scatter; the tiles of a prefill request are counted
// and placed by all 64 lanes of its owner's wave.  The static prefill
// assignment (first fit decreasing, the last wave) runs while the other
// waves scatter.  The barriers order LDS only: no thread reads another's
// work-list stores (the later kernels do), so none waits for them.  No host
// sync is needed: the later kernels read the counts from the workspace
// header.
#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kReqPerThread = 4;                           // requests a thread owns per chunk
constexpr int kChunkReqs = kPlanThreads * kReqPerThread;   // requests per chunk

struct Counts {
  int rows, prefill, reduce, slots, tail, reduce_long, stage;
};

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// makes this thread's global stores visible to the workgroup, i.e. waits
// until every work-list store in flight has completed (a memory round trip
// per barrier); no thread here reads another's global writes (only the
// later kernels do), so the barriers need not wait for them.
PKV_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive sum over the 64 lanes of a wave (every lane active): shifts by
// 1, 2, 4 and 8 inside each row of 16 lanes, then row 0's and row 1's last
// lanes broadcast into the rows after them (the gfx9 DPP row_bcast forms).
// Lanes a DPP move leaves without a source keep the 0 passed as `old`.
PKV_DEV int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan of N counters over the workgroup (every thread calls it):
// ex[c] = sum of v[c] over lower threads, tot[c] = the workgroup's sum.
// `lds` holds the wave totals; it is written before and read after the one
// barrier, so a caller that scans again into the same array must put a
// barrier between the two calls.
template <int N>
__device__ void block_scan(const int (&v)[N], int (&ex)[N], int (&tot)[N], int (*lds)[8]) {
  static_assert(N <= 8, "at most 8 counters");
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int inc[N];
#pragma unroll
  for (int c = 0; c < N; ++c) inc[c] = wave_incl_sum(v[c]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int c = 0; c < N; ++c) lds[w][c] = inc[c];
  }
  lds_barrier();
#pragma unroll
  for (int c = 0; c < N; ++c) {
    // lanes 0..15 hold the 16 wave totals; their inclusive sums inside row 0
    int t = lane < kPlanWaves ? lds[lane][c] : 0;
    t += __builtin_amdgcn_update_dpp(0, t, 0x111, 0xf, 0xf, false);
    t += __builtin_amdgcn_update_dpp(0, t, 0x112, 0xf, 0xf, false);
    t += __builtin_amdgcn_update_dpp(0, t, 0x114, 0xf, 0xf, false);
    t += __builtin_amdgcn_update_dpp(0, t, 0x118, 0xf, 0xf, false);
    const int before = w > 0 ? __builtin_amdgcn_readlane(t, w - 1) : 0;
    tot[c] = __builtin_amdgcn_readlane(t, kPlanWaves - 1);
    ex[c] = inc[c] - v[c] + before;
  }
}

// Buckets of the counting sorts that list work longest first.
constexpr int kPfBuckets = 4096;          // prefill tiles by KV tiles to read (clamped)
static_assert(kPfBuckets % kPlanThreads == 0, "buckets split evenly over the plan threads");
constexpr int kBucketsPerThread = kPfBuckets / kPlanThreads;
constexpr int kTailBuckets = kSplitBlocks; // partial partitions by block count

struct ReqInfo {
  int kind;  // 0 none, 1 decode row, 2 prefill tiles, 3 rows per query, 4 NaN rows
  int qs, ql, L, c, nparts, err;
};

// Request r's metadata (query_start_loc[r], query_start_loc[r + 1],
// seq_lens[r], num_computed_tokens[r]) checked and classified.
__device__ ReqInfo classify(const PlanParams& a, int r, int qs, int qe, int L, int c) {
  ReqInfo q{0, qs, qe - qs, L, c, 1, 0};
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

// Items a request contributes: full partitions or query rows (rows), its
// partial last partition (tail), prefill tiles, its reduce item (a short or
// a long row's) and the partial slots of its partitions.
__device__ Counts count_items(const PlanParams& a, const ReqInfo& q) {
  Counts m{0, 0, 0, 0, 0, 0, 0};
  if (q.kind == 1) {
    const bool partial_last = q.L % kSplitTokens != 0;
    m.rows = q.nparts - (partial_last ? 1 : 0);
    m.tail = partial_last ? 1 : 0;
    if (q.nparts > 1) {
      if (q.nparts <= a.reduce_short_parts)
        m.reduce = 1;
      else
        m.reduce_long = 1;
      m.slots = q.nparts;
    }
  } else if (q.kind == 2) {
    m.prefill = (q.ql + a.prefill_tile_rows - 1) / a.prefill_tile_rows;
    if (a.stage_capacity > 0) m.stage = (q.L + kBlock - 1) / kBlock;   // blocks its tiles read
  } else if (q.kind == 3 || q.kind == 4) {
    m.rows = q.ql;
  }
  return m;
}

// KV tiles (of 64 keys) a prefill tile starting at query row0 with `rows`
// rows reads: its bucket in the longest-first order.
__device__ int pf_bucket(int c, int row0, int rows) {
  const int kv_end = c + row0 + rows;
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
// directly; the rest are placed one by one, in a loop whose index and item
// cost are wave-uniform (scalar).  Lane s of the calling wave holds slot s's
// load and item count (loads stay below 2^24: at most 256 items of at most
// 4095 tiles); lane l also holds the costs and results of items l, l + 64,
// l + 128 and l + 192.  Writes slot_of[i] and the item's rank inside its
// slot, then the slot offsets (exclusive sums of the counts).
PKV_DEV int item_cost(int tiles) { return 10 * tiles + 50; }

PKV_DEV void assign_first_fit(const int* tiles, int n_in, int W_in, int* slot_of, int* rank_of, int* slot_start) {
  static_assert(kPfMaxStatic == 4 * kWave && kPfMaxSlots <= kWave, "four items per lane, one slot per lane");
  const int lane = threadIdx.x & (kWave - 1);
  const int n = __builtin_amdgcn_readfirstlane(n_in);
  const int W = __builtin_amdgcn_readfirstlane(W_in);
  int cst[4], res_slot[4], res_rank[4];
  int sum = 0, nbig = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = lane + kWave * s;
    cst[s] = i < n ? item_cost(tiles[i]) : 0;
    sum += cst[s];
  }
  const int total = __builtin_amdgcn_readlane(wave_incl_sum(sum), kWave - 1);
  const int cap = (total + W - 1) / W + 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) nbig += 2 * cst[s] > cap ? 1 : 0;
  const int big = __builtin_amdgcn_readlane(wave_incl_sum(nbig), kWave - 1);
  const int p = min(big, W);                        // items placed directly: item i in slot i
  const bool live = lane < W;
  const uint64_t live_mask = __ballot(live);
  int load = lane < p ? cst[0] : 0;
  int cnt = lane < p ? 1 : 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    res_slot[s] = 0;
    res_rank[s] = 0;
  }
  res_slot[0] = lane < p ? lane : 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j_end = min(n - kWave * s, kWave);
    for (int j = max(p - kWave * s, 0); j < j_end; ++j) {   // item kWave * s + j
      const int c = __builtin_amdgcn_readlane(cst[s], j);
      const int room = cap - c;   // scalar: one vector compare per item
      const uint64_t fits = __ballot(load <= room) & live_mask;
      int win;
      if (fits) {
        win = __builtin_ctzll(fits);
      } else {   // no slot has room: the emptiest one
        const int m = wave_max_i(live ? ((0xffffff - load) << 6) | (63 - lane) : -1);
        win = 63 - (__builtin_amdgcn_readfirstlane(m) & 63);
      }
      const int r = __builtin_amdgcn_readlane(cnt, win);
      if (lane == win) {
        load += c;
        cnt += 1;
      }
      if (lane == j) {
        res_slot[s] = win;
        res_rank[s] = r;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = lane + kWave * s;
    if (i < n) {
      slot_of[i] = res_slot[s];
      rank_of[i] = res_rank[s];
    }
  }
  // exclusive sums of the counts (W <= 64 lanes)
  const int cl = live ? cnt : 0;
  const int st = wave_incl_sum(cl) - cl;
  if (live) slot_start[lane] = st;
  if (lane == 0) slot_start[W] = n;   // W may be 64: no lane W
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams a) {
  __shared__ int err_acc, split_rows;
  __shared__ int scan_lds[3][kPlanWaves][8];
  __shared__ int pf_tiles[kPfMaxStatic], pf_slot_of[kPfMaxStatic], pf_rank[kPfMaxStatic];
  __shared__ int pf_start[kPfMaxSlots + 1];
  __shared__ int pf_off[kPfBuckets];
  __shared__ int tail_off[kTailBuckets];
  for (int i = threadIdx.x; i < kPfBuckets; i += kPlanThreads) pf_off[i] = 0;
  if (threadIdx.x < kTailBuckets) tail_off[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    err_acc = 0;
    split_rows = 0;
  }
  lds_barrier();

  const int nreq = a.num_reqs;
  const int nchunks = (nreq + kChunkReqs - 1) / kChunkReqs;
  // This thread's requests of the current chunk: rbeg .. rbeg + kown - 1.
  ReqInfo qi[kReqPerThread];
  int rbeg = 0, kown = 0;
  auto load_chunk = [&](int c0) {
    const int nc = min(kChunkReqs, nreq - c0);
    const int per = (nc + kPlanThreads - 1) / kPlanThreads;
    rbeg = c0 + (int)threadIdx.x * per;
    kown = max(0, min(per, c0 + nc - rbeg));
    // Every load is issued before any is used (one round trip); a thread
    // loads only its own requests (rbeg + kown <= nreq), and requests past
    // its run are classified as empty.
    int qs[kReqPerThread + 1], L[kReqPerThread], c[kReqPerThread];
#pragma unroll
    for (int k = 0; k <= kReqPerThread; ++k) qs[k] = k <= kown && kown > 0 ? a.qsl[rbeg + k] : 0;
#pragma unroll
    for (int k = 0; k < kReqPerThread; ++k) {
      L[k] = k < kown ? a.seq_lens[rbeg + k] : 0;
      c[k] = k < kown ? a.nct[rbeg + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < kReqPerThread; ++k)
      qi[k] = k < kown ? classify(a, rbeg + k, qs[k], qs[k + 1], L[k], c[k]) : ReqInfo{0, 0, 0, 0, 0, 1, 0};
  };

  // Pass 1: check requests, place decode rows (full partitions), reduce
  // items and per-query rows, count everything, and histogram the items that
  // are sorted.
  Counts base{0, 0, 0, 0, 0, 0, 0};
  int slot_first = 0;   // (single chunk) partial slot of this thread's first split row
  int stage_first = 0;  // (single chunk) first staged block of this thread's first prefill request
  for (int ch = 0; ch < nchunks; ++ch) {
    if (ch > 0) lds_barrier();   // scan_lds[0] is read by every thread before it is rewritten
    load_chunk(ch * kChunkReqs);
    int own[7] = {0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < kReqPerThread; ++k) {
      const Counts m = count_items(a, qi[k]);
      own[0] += m.rows;
      own[1] += m.prefill;
      own[2] += m.reduce;
      own[3] += m.slots;
      own[4] += m.tail;
      own[5] += m.reduce_long;
      own[6] += m.stage;
    }
    int ex[7], tot[7];
    block_scan<7>(own, ex, tot, scan_lds[0]);
    stage_first = base.stage + ex[6];
    int rowpos = base.rows + ex[0], redpos = base.reduce + ex[2], slotpos = base.slots + ex[3];
    int redpos_l = base.reduce_long + ex[5];   // long rows: from the end of the list
    slot_first = slotpos;
    const bool sorted_fit = base.tail + tot[4] <= a.cap_row_items && base.prefill + tot[1] <= a.cap_prefill_items;
    int err = 0;
    bool pf_req[kReqPerThread];   // prefill requests whose tiles go into the histogram
#pragma unroll
    for (int k = 0; k < kReqPerThread; ++k) {
      pf_req[k] = false;
      if (k >= kown) continue;
      const ReqInfo q = qi[k];
      const int r = rbeg + k;
      const Counts m = count_items(a, q);
      err |= q.err;
      const bool fits = sorted_fit && rowpos + m.rows <= a.cap_row_items && redpos + m.reduce <= a.cap_reduce &&
                        redpos_l + m.reduce_long <= a.cap_reduce && slotpos + m.slots <= a.cap_slots;
      if (!fits) {
        err |= PKV_DEVERR_CAPACITY;
      } else if (q.kind == 1) {
        for (int p = 0; p < m.rows; ++p)
          a.row_items[rowpos + p] = make_int4(q.qs, r, q.nparts == 1 ? kWholeRow : p, q.nparts == 1 ? -1 : slotpos);
        if (m.tail) atomicAdd(&tail_off[(q.L % kSplitTokens + kBlock - 1) / kBlock - 1], 1);
        if (m.reduce) a.reduce_items[redpos] = make_int4(q.qs, r, q.nparts, slotpos);
        if (m.reduce_long) {
          a.reduce_items[a.cap_reduce - 1 - redpos_l] = make_int4(q.qs, r, q.nparts, slotpos);
          if (q.nparts > 2 * a.reduce_short_parts) atomicAdd(&split_rows, 1);
        }
      } else if (q.kind == 2) {
        pf_req[k] = true;
      } else if (q.kind == 3 || q.kind == 4) {
        const int z = q.kind == 3 ? kWholeRow : kNanRow;
        for (int i = 0; i < q.ql; ++i) a.row_items[rowpos + i] = make_int4(q.qs + i, r, z, -1);
      }
      rowpos += m.rows;
      redpos += m.reduce;
      redpos_l += m.reduce_long;
      slotpos += m.slots;
    }
    // A prefill request's tiles are histogrammed by the whole wave, one tile
    // per lane (a request may have thousands; its owner alone would count
    // them one by one).
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 0; k < kReqPerThread; ++k) {
      for (uint64_t m = __ballot(pf_req[k]); m; m &= m - 1) {
        const int src = __builtin_ctzll(m);
        const int ql = __builtin_amdgcn_readlane(qi[k].ql, src), c = __builtin_amdgcn_readlane(qi[k].c, src);
        const int tr = a.prefill_tile_rows;
        for (int row0 = lane * tr; row0 < ql; row0 += kWave * tr)
          atomicAdd(&pf_off[pf_bucket(c, row0, min(tr, ql - row0))], 1);
      }
    }
    if (err) atomicOr(&err_acc, err);
    base.rows += tot[0];
    base.prefill += tot[1];
    base.reduce += tot[2];
    base.slots += tot[3];
    base.tail += tot[4];
    base.reduce_long += tot[5];
    base.stage += tot[6];
  }
  const bool over = base.rows > a.cap_row_items || base.tail > a.cap_row_items ||
                    base.prefill > a.cap_prefill_items || base.reduce + base.reduce_long > a.cap_reduce ||
                    base.slots > a.cap_slots;
  // 8-bit cache: the prefill reads its blocks from the staging area when they
  // all fit there (each is dequantised once, instead of once per prefill tile
  // that reads it)
  const bool staged = !over && base.stage > 0 && base.stage <= a.stage_capacity;
  // Bucket offsets, longest bucket first: thread t owns the 4 buckets at
  // descending positions 4t .. 4t+3 of the prefill list and writes the tile
  // count of each of their positions below kPfMaxStatic (the first-fit
  // input: items of one bucket cost the same, so the assignment does not
  // depend on which of them the scatter puts where); thread 0 also does the
  // 32 tail buckets.  (Skipped, like the scatter, when nothing is sorted:
  // base is the same in every thread.)
  const bool sorted_work = base.prefill > 0 || base.tail > 0;
  lds_barrier();   // the histograms are complete
  if (sorted_work) {
    int n[kBucketsPerThread], local[1] = {0}, run[1], tot[1];
#pragma unroll
    for (int i = 0; i < kBucketsPerThread; ++i) {
      n[i] = pf_off[kPfBuckets - 1 - (kBucketsPerThread * threadIdx.x + i)];
      local[0] += n[i];
    }
    block_scan<1>(local, run, tot, scan_lds[1]);
    int off = run[0];
#pragma unroll
    for (int i = 0; i < kBucketsPerThread; ++i) {
      const int b = kPfBuckets - 1 - (kBucketsPerThread * threadIdx.x + i);
      pf_off[b] = off;
      for (int q = off; q < min(off + n[i], kPfMaxStatic); ++q) pf_tiles[q] = b;
      off += n[i];
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
  lds_barrier();

  // Static prefill assignment when it is small enough to build here (the last
// wave, whose threads own the last requests and usually none);
  // otherwise the prefill kernel takes items from per-head queues.
  const int npf = base.prefill;
  const bool pf_static = !over && npf > 0 && npf <= kPfMaxStatic && a.prefill_slots > 0 &&
                         a.prefill_slots <= kPfMaxSlots;
  if (pf_static && threadIdx.x >= kPlanThreads - kWave) assign_first_fit(pf_tiles, npf, a.prefill_slots, pf_slot_of, pf_rank, pf_start);

  // Pass 2: scatter the sorted items (order inside a bucket is irrelevant:
  // an item's result does not depend on which worker computes it).  With one
  // chunk every thread still holds its requests and the partial slot of its
  // first split row; otherwise each chunk is loaded and scanned again.
  if (!over && sorted_work) {
    int slot_base = 0, stage_base = 0;
    for (int ch = 0; ch < nchunks; ++ch) {
      int sp = slot_first, stp = stage_first;
      if (nchunks > 1) {
        if (ch > 0) lds_barrier();   // scan_lds[2] is read by every thread before it is rewritten
        load_chunk(ch * kChunkReqs);
        int own[2] = {0, 0}, ex[2], tot[2];
#pragma unroll
        for (int k = 0; k < kReqPerThread; ++k) {
          const Counts m = count_items(a, qi[k]);
          own[0] += m.slots;
          own[1] += m.stage;
        }
        block_scan<2>(own, ex, tot, scan_lds[2]);
        sp = slot_base + ex[0];
        slot_base += tot[0];
        stp = stage_base + ex[1];
        stage_base += tot[1];
      }
      const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
      for (int k = 0; k < kReqPerThread; ++k) {
        const ReqInfo q = qi[k];   // empty past this thread's run
        const int r = rbeg + k;
        if (q.kind == 1 && q.L % kSplitTokens != 0) {
          const int nb = (q.L % kSplitTokens + kBlock - 1) / kBlock;
          const int pos = atomicAdd(&tail_off[nb - 1], 1);
          a.row_items_tail[pos] = q.nparts == 1 ? make_int4(q.qs, r, kWholeRow, -1)
                                                : make_int4(q.qs, r, q.nparts - 1, sp);
        }
        // a prefill request's tiles are placed by the whole wave, one per lane
        for (uint64_t m = __ballot(q.kind == 2); m; m &= m - 1) {
          const int src = __builtin_ctzll(m);
          const int qs = __builtin_amdgcn_readlane(q.qs, src), ql = __builtin_amdgcn_readlane(q.ql, src);
          const int c = __builtin_amdgcn_readlane(q.c, src), rq = __builtin_amdgcn_readlane(r, src);
          const int tr = a.prefill_tile_rows;
          for (int row0 = lane * tr; row0 < ql; row0 += kWave * tr) {
            const int rows = min(tr, ql - row0);
            const int pos = atomicAdd(&pf_off[pf_bucket(c, row0, rows)], 1);
            a.prefill_items[pos] = make_int4(rq, qs + row0, rows, c - qs);
          }
          if (staged) {   // its staging: block kb -> staged block sb0 + kb, sources checked
            const int sb0 = __builtin_amdgcn_readlane(stp, src);
            const int nb = (__builtin_amdgcn_readlane(q.L, src) + kBlock - 1) / kBlock;
            const size_t row = (size_t)rq * a.max_blocks_per_req;
            for (int kb = lane; kb < nb; kb += kWave) {
              const int id = a.block_table[row + kb];
              const bool ok = id >= 0 && id < a.num_blocks;
              a.stage_src[sb0 + kb] = ok ? id : 0;
              a.stage_bt[row + kb] = ok ? sb0 + kb : -1;
            }
          }
        }
        if (q.kind == 1 && q.nparts > 1) sp += q.nparts;
        if (q.kind == 2) stp += count_items(a, q).stage;
      }
    }
  }
  lds_barrier();
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
    a.hdr[kHdrReduceItems] = over ? 0 : base.reduce + base.reduce_long;
    a.hdr[kHdrReduceShort] = over ? 0 : base.reduce;
    a.hdr[kHdrReduceSplit] = over ? 0 : split_rows;
    a.hdr[kHdrPrefillStaged] = staged ? 1 : 0;
    a.hdr[kHdrStagedBlocks] = staged ? base.stage : 0;
    a.hdr[kHdrSlots] = over ? 0 : base.slots;
  }
}

}  // namespace

int launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
