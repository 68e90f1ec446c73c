// Internal launch interface between the host entry points (pkv_api.cpp) and
// the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_kv.h"

namespace pkv {

// Status helpers shared by the host entry points: set the calling thread's
// error detail (printf format with up to three long long arguments) and
// return `status`; ok() clears the detail and returns PKV_OK.
int fail(int status, const char* fmt, long long a = 0, long long b = 0, long long c = 0);
int ok();

struct PlanParams {
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* nct;
  int32_t num_reqs;
  int64_t num_tokens;
  int32_t max_query_len, max_seq_len, max_blocks_per_req;
  int32_t split_decode;      // decode rows may be split into partitions
  int32_t mfma_prefill;      // query_len > 1 requests go to the prefill kernel
  int32_t prefill_tile_rows; // query rows per prefill tile
  int32_t prefill_slots;     // prefill workgroups per kv head (the prefill grid / num_kv_heads)
  int32_t reduce_short_parts;  // split rows of at most this many partitions are "short" reduce items
  // 8-bit cache, prefill on the matrix cores: staging of the prefill blocks
  // (stage_capacity 0: none).  stage_bt gets block_table's shape; the rows of
  // prefill requests are written (kb -> staged block, -1 for an id outside
  // the pool), stage_src[staged block] = the cache block it copies.
  int64_t stage_capacity;
  int32_t* stage_bt;
  int32_t* stage_src;
  const int32_t* block_table;
  int32_t num_blocks;
  int32_t* hdr;
  int4* row_items;
  int4* row_items_tail;
  int4* prefill_items;
  int4* reduce_items;
  int32_t* pf_order;         // static prefill assignment: item indices slot by slot
  int32_t* pf_slot_start;    // [prefill_slots + 1] offsets of each slot's items in pf_order
  int64_t cap_row_items, cap_prefill_items, cap_reduce, cap_slots;
};

struct RowParams {
  void* out;
  const void* q;
  const void* cache;  // layer base: K half then V half
  const int32_t* block_table;
  const int32_t* qsl;
  const int32_t* nct;
  const int4* items;       // first region (long items)
  const int4* items_tail;  // second region
  int32_t* hdr;
  float* part_o;
  float2* part_ml;
  int32_t* err;
  float scale_log2;  // scale * log2(e)
  int32_t num_q_heads, num_kv_heads, group, head_groups, num_blocks, max_blocks_per_req;
};

struct ReduceParams {
  void* out;
  const int4* items;       // short rows from the front, long rows from position cap_reduce - 1 down
  const int32_t* hdr;
  const float* part_o;
  const float2* part_ml;
  int32_t num_q_heads;
  int64_t cap_reduce;
};

struct PrefillParams {
  void* out;
  const void* q;
  const void* cache;
  const int32_t* block_table;
  const int4* items;       // tiles (request, first query token, rows, computed - first token)
  int32_t* hdr;
  int32_t* err;
  const int32_t* pf_order;       // per-slot item lists, used when hdr[kHdrPrefillStatic] is 1
  const int32_t* pf_slot_start;
  const float* kv_scales;  // 8-bit cache: [2][num_blocks][num_kv_heads][16] scales; else nullptr
  int32_t kv_fp8;          // 8-bit cache codes: 0 INT8, 1 OCP E4M3
  int32_t staged;          // runs only if hdr[kHdrPrefillStaged] equals this (1: over the staging area)
  float scale_log2;
  int32_t num_q_heads, num_kv_heads, group, num_blocks, max_blocks_per_req;
};

int launch_kv_write(const void* k, const void* v, const int64_t* slot_mapping, void* cache,
                    int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, int32_t elem_bytes, int32_t* device_error,
                    hipStream_t stream);
struct RopeParams {
  void* q;                      // [T][num_q_heads][head_dim] or nullptr, rotated in place
  const void* k;
  const void* v;
  const int64_t* positions;
  const float* cos_sin_cache;   // [max_position][rotary_dim]
  const int64_t* slot_mapping;
  void* cache;
  int64_t num_tokens;
  int32_t max_position, rotary_dim, is_neox;
  int32_t num_q_heads, num_blocks, num_kv_heads, head_dim;
  int32_t* device_error;
};
int launch_kv_write_rope(const RopeParams& p, bool bf16, hipStream_t stream);

int launch_kv_write_i8(const void* k, const void* v, const int64_t* slot_mapping, void* cache, float* scales,
                       int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, bool bf16,
                       bool fp8, int32_t* device_error, hipStream_t stream);
// Row kernels over an 8-bit (INT8 or FP8 E4M3) cache (decode_i8.hip); query
// heads per wave:
int max_group_regs_i8(int32_t dtype);
int launch_rows_i8(const RowParams& p, const float* kv_scales, int32_t dtype, int32_t head_dim, bool fp8,
                   int64_t bound_waves, int cus, hipStream_t stream);

int launch_kv_copy_blocks(void* cache, const int32_t* copies, int32_t num_copies, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes, int32_t* device_error,
                          hipStream_t stream);
int launch_plan(const PlanParams& p, hipStream_t stream);
// Dequantise the step's prefill blocks into the staging area (a no-op unless
// the plan staged them).
struct StageParams {
  const void* cache;        // 8-bit cache layer: K codes then V codes
  const float* kv_scales;   // [2][num_blocks][num_kv_heads][16]
  const int32_t* src;       // stage_src
  void* staged;             // bf16 [2][capacity][16][num_kv_heads][head_dim]
  const int32_t* hdr;
  int64_t capacity;
  int32_t num_blocks, num_kv_heads, head_dim, fp8;
};
int launch_stage(const StageParams& p, int64_t grid, hipStream_t stream);
// bound_waves: upper bound on row work items (one wave each); cus: compute units.
// Query heads of a group that one row wave handles (wider groups run as
// head_groups waves over the same blocks).
int max_group_regs(int32_t dtype, int32_t group, int32_t head_dim);
int launch_rows(const RowParams& p, int32_t dtype, int32_t head_dim, int64_t bound_waves, int cus,
                hipStream_t stream);
int launch_reduce(const ReduceParams& p, int32_t dtype, int32_t head_dim, int64_t grid,
                  hipStream_t stream);
// Partitions of the longest row the merge takes as a "short" row (four query
// heads per wave and pass).
int reduce_short_parts(int32_t head_dim);
int prefill_tile_rows(int32_t group);
int launch_prefill(const PrefillParams& p, int32_t head_dim, int64_t grid, hipStream_t stream);

}  // namespace pkv
