// Step planning on the device: from query_start_loc, seq_lens and
// num_computed_tokens, check each request and turn the step into work lists.
//
// Continuous batching ("AI Infra入门干货总结：大模型是如何高效推理的",
// section "连续批处理") schedules, per request, the tokens between
// num_computed_tokens and num_tokens, with no separate prefill and decode
// phases; one step therefore mixes single-token decodes and multi-token
// prefill chunks.  This kernel sorts them:
//   query_len == 1  -> decode row; split into 512-token partitions when the
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

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams a) {
  __shared__ int err_acc;
  if (threadIdx.x == 0) err_acc = 0;
  __syncthreads();
  Counts base{0, 0, 0, 0, 0};
  const int64_t T = a.num_tokens;
  for (int r0 = 0; r0 < a.num_reqs; r0 += kPlanThreads) {
    const int r = r0 + threadIdx.x;
    int kind = 0;  // 0 none, 1 decode row, 2 prefill tiles, 3 rows per query, 4 NaN rows
    int qs = 0, ql = 0, nparts = 1, L = 0;
    int err = 0;
    if (r < a.num_reqs) {
      qs = a.qsl[r];
      const int qe = a.qsl[r + 1];
      ql = qe - qs;
      L = a.seq_lens[r];
      const int c = a.nct[r];
      const bool qsl_ok = qs >= 0 && ql >= 0 && (int64_t)qe <= T && (r > 0 || qs == 0);
      if (!qsl_ok) {
        err |= PKV_DEVERR_QSL;
      } else if (c < 0 || L != c + ql) {
        err |= PKV_DEVERR_SEQ_LEN;
        kind = 4;
      } else if (ql > a.max_query_len || L > a.max_seq_len ||
                 L > a.max_blocks_per_req * kBlock) {
        err |= PKV_DEVERR_LIMITS;
        kind = 4;
      } else if (ql == 1) {
        kind = 1;
        nparts = a.split_decode ? (L + kSplitTokens - 1) / kSplitTokens : 1;
      } else if (ql > 1) {
        kind = a.mfma_prefill ? 2 : 3;
      }
      if (kind == 4 && ql == 0) kind = 0;
    }
    // Row items go to two regions so that workers claim the long ones first:
    // "rows" holds full 512-token partitions and whole rows, "tail" the
    // partial last partition of each decode row.
    Counts mine{0, 0, 0, 0, 0};
    const bool partial_last = kind == 1 && L % kSplitTokens != 0;
    if (kind == 1) {
      mine.rows = nparts - (partial_last ? 1 : 0);
      mine.tail = partial_last ? 1 : 0;
      if (nparts > 1) {
        mine.reduce = 1;
        mine.slots = nparts;
      }
    } else if (kind == 2) {
      mine.prefill = (ql + a.prefill_tile_rows - 1) / a.prefill_tile_rows;
    } else if (kind == 3 || kind == 4) {
      mine.rows = ql;
    }
    Counts tot;
    Counts ex = block_exclusive_scan(mine, &tot);
    ex.rows += base.rows;
    ex.prefill += base.prefill;
    ex.reduce += base.reduce;
    ex.slots += base.slots;
    ex.tail += base.tail;
    const bool fits = ex.rows + mine.rows <= a.cap_row_items &&
                      ex.tail + mine.tail <= a.cap_row_items &&
                      ex.prefill + mine.prefill <= a.cap_prefill_items &&
                      ex.reduce + mine.reduce <= a.cap_reduce &&
                      ex.slots + mine.slots <= a.cap_slots;
    if (!fits) {
      err |= PKV_DEVERR_CAPACITY;
    } else if (kind == 1) {
      for (int p = 0; p < nparts; ++p) {
        const int4 it = make_int4(qs, r, nparts == 1 ? kWholeRow : p, nparts == 1 ? -1 : ex.slots);
        if (partial_last && p == nparts - 1)
          a.row_items_tail[ex.tail] = it;
        else
          a.row_items[ex.rows + p] = it;
      }
      if (nparts > 1) a.reduce_items[ex.reduce] = make_int4(qs, r, nparts, ex.slots);
    } else if (kind == 2) {
      // Latest tiles first: they see the most keys (longest work first).
      for (int j = 0; j < mine.prefill; ++j) {
        const int tile = mine.prefill - 1 - j;
        const int row0 = tile * a.prefill_tile_rows;
        const int rows = min(a.prefill_tile_rows, ql - row0);
        a.prefill_items[ex.prefill + j] = make_int4(r, row0, rows, 0);
      }
    } else if (kind == 3 || kind == 4) {
      const int z = kind == 3 ? kWholeRow : kNanRow;
      for (int i = 0; i < ql; ++i) a.row_items[ex.rows + i] = make_int4(qs + i, r, z, -1);
    }
    if (err) atomicOr(&err_acc, err);
    base.rows += tot.rows;
    base.prefill += tot.prefill;
    base.reduce += tot.reduce;
    base.slots += tot.slots;
    base.tail += tot.tail;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool over = base.rows > a.cap_row_items || base.tail > a.cap_row_items ||
                      base.prefill > a.cap_prefill_items ||
                      base.reduce > a.cap_reduce || base.slots > a.cap_slots;
    // On overflow nothing past the capacity was written; run no work at all.
    a.hdr[kHdrError] = err_acc | (over ? PKV_DEVERR_CAPACITY : 0);
    a.hdr[kHdrRowItems] = over ? 0 : base.rows + base.tail;
    a.hdr[kHdrRowHead] = over ? 0 : base.rows;
    a.hdr[kHdrPrefillItems] = over ? 0 : base.prefill;
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
