// Host side of libpagedkv: the extern "C" entry points declared in
// include/paged_kv.h.  Arguments are checked here before anything is
// enqueued; the kernels are launched on the caller's stream with no
// allocation and no synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace {
thread_local std::string g_detail;
}  // namespace

namespace pkv {

int fail(int status, const char* fmt, long long a, long long b, long long c) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  g_detail = buf;
  return status;
}

int ok() {
  g_detail.clear();
  return PKV_OK;
}

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::ok;

int elem_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : dtype == PKV_F32 ? 4 : 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Compute units of the current device, cached per device id.
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The stream the prefill kernel runs on beside the caller's stream, one per
// device, created on first use with the default priority and not
// synchronising with the null stream.  The prefill (bound by the matrix
// cores) and the decode rows (bound by HBM) of one step are independent;
// on a second stream the rows' workgroups take the CUs that the prefill's
// last workgroups leave free.  Used for the 8-bit caches, where it measured
// 1.3% faster on the mixed step; with a bf16 cache it measured 0.3% slower
// (the row kernels' fixed item order lets little of the prefill's tail be
// reclaimed, and running both draws more power).  nullptr when it cannot be
// created (the step then runs on the caller's stream alone).
constexpr int kMaxSideDevices = 64;
struct SideStream {
  std::once_flag once;
  hipStream_t s = nullptr;
};
SideStream g_side[kMaxSideDevices];

hipStream_t side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& e = g_side[dev];
  std::call_once(e.once, [&e] {
    hipStream_t st = nullptr;
    e.s = hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess ? st : nullptr;
  });
  return e.s;
}

// A fork of the step onto the side stream: the side stream waits for what the
// caller's stream has enqueued so far, and join() makes the caller's stream
// wait for what was enqueued on the side stream since.  The two events are
// the call's own (created here, released by join, which every path out of the
// call runs), so concurrent calls never share one.
struct Fork {
  hipStream_t main = nullptr, side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool begin(hipStream_t s) {
    main = s;
    side = side_stream();
    if (side == nullptr || side == s) return false;
    if (hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming) != hipSuccess) return release(), false;
    if (hipEventCreateWithFlags(&ev_join, hipEventDisableTiming) != hipSuccess) return release(), false;
    if (hipEventRecord(ev_fork, main) != hipSuccess || hipStreamWaitEvent(side, ev_fork, 0) != hipSuccess)
      return release(), false;
    return true;
  }
  void release() {
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
    ev_fork = ev_join = nullptr;
    side = nullptr;
  }
  // the caller's stream waits for the side stream's work (0 on success)
  int join() {
    if (side == nullptr) return 0;
    const bool ok = hipEventRecord(ev_join, side) == hipSuccess && hipStreamWaitEvent(main, ev_join, 0) == hipSuccess;
    release();
    return ok ? 0 : 1;
  }
  ~Fork() { (void)join(); }
};

// Prefill chunks with bf16 q run on the MFMA tile kernel: over a bf16 cache
// at head_dim 64 or 128, over an 8-bit cache at head_dim 128.  Other prefill
// rows (fp32, 8-bit caches at head_dim 64) go through the row kernel, one
// query row at a time.
bool prefill_on_mfma(int32_t dtype, int32_t head_dim, bool kv8) {
  return dtype == PKV_BF16 && (head_dim == 128 || (head_dim == 64 && !kv8));
}

int64_t tile_rows_for(int32_t dtype, int32_t head_dim, int32_t group, bool kv8) {
  return prefill_on_mfma(dtype, head_dim, kv8) ? pkv::prefill_tile_rows(group) : 1;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer argument";
    case PKV_ERR_DIMS: return "invalid or unsupported size";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_METADATA: return "inconsistent metadata";
    case PKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

const char* pkv_last_error_detail(void) { return g_detail.c_str(); }

int paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                   void* kv_cache_layer, int64_t num_tokens, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   int32_t* device_error, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_tokens < 0) return fail(PKV_ERR_DIMS, "num_tokens %lld < 0", num_tokens);
  if (num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_DIMS, "num_blocks %lld, num_kv_heads %lld", num_blocks, num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_DIMS, "head_dim %lld not 64/128", head_dim);
  if (kv_cache_layer == nullptr) return fail(PKV_ERR_NULL, "kv_cache_layer is NULL");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v or slot_mapping is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kv_cache_layer, 16) || !aligned(slot_mapping, 8))
    return fail(PKV_ERR_ALIGN, "k, v, cache must be 16-byte aligned, slot_mapping 8-byte");
  if (pkv::launch_kv_write(k, v, slot_mapping, kv_cache_layer, num_tokens, num_blocks, num_kv_heads,
                           head_dim, eb, device_error, (hipStream_t)stream))
    return fail(PKV_ERR_LAUNCH, "kv_write launch: %lld", (long long)hipGetLastError());
  return ok();
}

int paged_kv_write_rope(void* q, const void* k, const void* v, const int64_t* positions,
                        const float* cos_sin_cache, int32_t max_position, int32_t rotary_dim,
                        int32_t is_neox, const int64_t* slot_mapping, void* kv_cache_layer,
                        int64_t num_tokens, int32_t num_q_heads, int32_t num_blocks,
                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t* device_error, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_tokens < 0) return fail(PKV_ERR_DIMS, "num_tokens %lld < 0", num_tokens);
  if (num_blocks <= 0 || num_kv_heads <= 0 || (q != nullptr && num_q_heads <= 0))
    return fail(PKV_ERR_DIMS, "num_blocks %lld, num_kv_heads %lld, num_q_heads %lld", num_blocks, num_kv_heads,
                num_q_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_DIMS, "head_dim %lld not 64/128", head_dim);
  if (rotary_dim < 2 || rotary_dim > head_dim || rotary_dim % 2 != 0 || max_position <= 0)
    return fail(PKV_ERR_DIMS, "rotary_dim %lld, max_position %lld", rotary_dim, max_position);
  if (kv_cache_layer == nullptr) return fail(PKV_ERR_NULL, "kv_cache_layer is NULL");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !positions || !cos_sin_cache)
    return fail(PKV_ERR_NULL, "k, v, slot_mapping, positions or cos_sin_cache is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kv_cache_layer, 16) || (q && !aligned(q, 16)) ||
      !aligned(slot_mapping, 8) || !aligned(positions, 8) || !aligned(cos_sin_cache, 4))
    return fail(PKV_ERR_ALIGN, "q, k, v, cache must be 16-byte aligned, slot_mapping / positions 8-byte");
  pkv::RopeParams p{q, k, v, positions, cos_sin_cache, slot_mapping, kv_cache_layer, num_tokens,
                    max_position, rotary_dim, is_neox != 0, num_q_heads, num_blocks, num_kv_heads, head_dim,
                    device_error};
  if (pkv::launch_kv_write_rope(p, dtype == PKV_BF16, (hipStream_t)stream))
    return fail(PKV_ERR_LAUNCH, "kv_write_rope launch: %lld", (long long)hipGetLastError());
  return ok();
}

int paged_kv_copy_blocks(void* kv_cache_layer, const int32_t* copies, int32_t num_copies,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         int32_t* device_error, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_copies < 0) return fail(PKV_ERR_DIMS, "num_copies %lld < 0", num_copies);
  if (num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_DIMS, "num_blocks %lld, num_kv_heads %lld", num_blocks, num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_DIMS, "head_dim %lld not 64/128", head_dim);
  if (kv_cache_layer == nullptr) return fail(PKV_ERR_NULL, "kv_cache_layer is NULL");
  if (num_copies == 0) return ok();
  if (!copies) return fail(PKV_ERR_NULL, "copies is NULL");
  if (!aligned(kv_cache_layer, 16) || !aligned(copies, 4))
    return fail(PKV_ERR_ALIGN, "cache must be 16-byte aligned, copies 4-byte");
  if (pkv::launch_kv_copy_blocks(kv_cache_layer, copies, num_copies, num_blocks, num_kv_heads, head_dim, eb,
                                 device_error, (hipStream_t)stream))
    return fail(PKV_ERR_LAUNCH, "copy_blocks launch: %lld", (long long)hipGetLastError());
  return ok();
}

static size_t workspace_size_tiles(int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                                         int32_t head_dim, int32_t max_query_len,
                                         int32_t max_seq_len, int64_t tile_rows) {
  if (num_reqs < 0 || num_tokens < 0 || num_q_heads <= 0 || head_dim <= 0 || max_query_len < 0 ||
      max_seq_len < 0)
    return 0;
  return pkv::ws_layout(num_reqs, num_tokens, num_q_heads, head_dim, max_query_len, max_seq_len,
                        tile_rows)
      .total;
}

size_t paged_attention_workspace_size(int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_query_len,
                                      int32_t max_seq_len) {
  // Tile count bound with one-row tiles covers every prefill tiling.
  return workspace_size_tiles(num_reqs, num_tokens, num_q_heads, head_dim,
                                           max_query_len, max_seq_len, 1);
}

size_t paged_attention_staging_bytes(int32_t num_reqs, int32_t max_blocks_per_req, int32_t num_kv_heads,
                                     int32_t head_dim, int64_t prefill_blocks) {
  if (num_reqs < 0 || max_blocks_per_req < 0 || num_kv_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
      prefill_blocks < 0)
    return 0;
  if (prefill_blocks == 0) return 0;
  // covers the alignments stage_layout() applies after the workspace's own size
  return 256 + pkv::align_up(sizeof(int32_t) * (size_t)num_reqs * (size_t)max_blocks_per_req, 256) +
         pkv::align_up(sizeof(int32_t) * (size_t)prefill_blocks, 256) +
         (size_t)prefill_blocks * (size_t)pkv::stage_block_bytes(num_kv_heads, head_dim) + 1024;
}

static int attention_impl(void* out, const void* q, const void* kv_cache_layer,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                          float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                          int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                          int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* phase_events, const float* kv_scales = nullptr, bool fp8 = false,
                          bool overlap = false) {
  const bool i8 = kv_scales != nullptr;   // 8-bit cache (INT8, or E4M3 when fp8) + per-(token, head) scales
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_reqs < 0 || num_tokens < 0)
    return fail(PKV_ERR_DIMS, "num_reqs %lld, num_tokens %lld", num_reqs, num_tokens);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_kv_heads > pkv::kMaxKvHeads ||
      num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 16)
    return fail(PKV_ERR_DIMS, "num_q_heads %lld / num_kv_heads %lld", num_q_heads, num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_DIMS, "head_dim %lld not 64/128", head_dim);
  if (num_blocks <= 0 || max_blocks_per_req <= 0 || max_query_len < 0 || max_seq_len < 0)
    return fail(PKV_ERR_DIMS, "num_blocks %lld, max_blocks_per_req %lld, limits", num_blocks,
                max_blocks_per_req);
  if (!std::isfinite(scale)) return fail(PKV_ERR_DIMS, "scale is not finite");
  if (!out && num_tokens > 0) return fail(PKV_ERR_NULL, "out is NULL");
  if (!q && num_tokens > 0) return fail(PKV_ERR_NULL, "q is NULL");
  if (!kv_cache_layer || !workspace || !query_start_loc)
    return fail(PKV_ERR_NULL, "kv_cache_layer, workspace or query_start_loc is NULL");
  if (num_reqs > 0 && (!block_table || !seq_lens || !num_computed_tokens))
    return fail(PKV_ERR_NULL, "block_table, seq_lens or num_computed_tokens is NULL");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(kv_cache_layer, 16) ||
      !aligned(workspace, 256))
    return fail(PKV_ERR_ALIGN, "out, q, cache need 16-byte alignment, workspace 256-byte");
  if ((int64_t)num_blocks * pkv::kBlock * num_kv_heads * head_dim * (i8 ? 1 : eb) > (int64_t)1 << 46)
    return fail(PKV_ERR_DIMS, "cache too large");
  if (i8 && !aligned(kv_scales, 4)) return fail(PKV_ERR_ALIGN, "kv_scales needs 4-byte alignment");

  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t tile_rows = tile_rows_for(dtype, head_dim, group, i8);
  const pkv::WsLayout ws =
      pkv::ws_layout(num_reqs, num_tokens, num_q_heads, head_dim, max_query_len, max_seq_len, tile_rows);
  if (workspace_bytes < ws.total)
    return fail(PKV_ERR_WORKSPACE, "workspace %lld bytes < %lld needed", (long long)workspace_bytes,
                (long long)ws.total);

  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int phase, int end) {
    if (phase_events && phase_events[2 * phase + end])
      (void)hipEventRecord((hipEvent_t)phase_events[2 * phase + end], s);
  };
  char* wsb = (char*)workspace;
  int32_t* hdr = (int32_t*)wsb;

  pkv::PlanParams pp{};
  pp.qsl = query_start_loc;
  pp.seq_lens = seq_lens;
  pp.nct = num_computed_tokens;
  pp.num_reqs = num_reqs;
  pp.num_tokens = num_tokens;
  pp.max_query_len = max_query_len;
  pp.max_seq_len = max_seq_len;
  pp.max_blocks_per_req = max_blocks_per_req;
  pp.split_decode = 1;
  pp.mfma_prefill = prefill_on_mfma(dtype, head_dim, i8) ? 1 : 0;
  pp.prefill_tile_rows = (int32_t)tile_rows;
  // One 8-wave prefill workgroup per CU; the grid is a multiple of the kv
  // head count so every workgroup owns one head (slot = blockIdx / heads).
  const int cus = num_cus();
  const int64_t pf_per_head =
      std::max<int64_t>(1, std::min<int64_t>(ws.cap_prefill_items, (int64_t)cus / num_kv_heads));
  pp.prefill_slots = (int32_t)pf_per_head;
  pp.reduce_short_parts = pkv::reduce_short_parts(head_dim);
  pp.block_table = block_table;
  pp.num_blocks = num_blocks;
  // 8-bit cache, prefill on the matrix cores: workspace past ws.total stages
  // the step's prefill blocks in bf16 when they fit (see stage.hip).
  const pkv::StageLayout stl =
      i8 && pp.mfma_prefill ? pkv::stage_layout(ws.total, workspace_bytes, num_reqs, max_blocks_per_req,
                                                num_kv_heads, head_dim)
                            : pkv::StageLayout{};
  pp.stage_capacity = stl.capacity;
  pp.stage_bt = stl.capacity > 0 ? (int32_t*)(wsb + stl.bt) : nullptr;
  pp.stage_src = stl.capacity > 0 ? (int32_t*)(wsb + stl.src) : nullptr;
  pp.hdr = hdr;
  pp.row_items = (int4*)(wsb + ws.row_items);
  pp.row_items_tail = (int4*)(wsb + ws.row_items_tail);
  pp.prefill_items = (int4*)(wsb + ws.prefill_items);
  pp.reduce_items = (int4*)(wsb + ws.reduce_items);
  pp.pf_order = (int32_t*)(wsb + ws.pf_order);
  pp.pf_slot_start = (int32_t*)(wsb + ws.pf_slot_start);
  pp.cap_row_items = ws.cap_row_items;
  pp.cap_prefill_items = ws.cap_prefill_items;
  pp.cap_reduce = ws.cap_reduce;
  pp.cap_slots = ws.cap_slots;
  mark(PKV_PHASE_PLAN, 0);
  if (pkv::launch_plan(pp, s)) return fail(PKV_ERR_LAUNCH, "plan launch failed");
  mark(PKV_PHASE_PLAN, 1);

  const float scale_log2 = scale * 1.4426950408889634f;
  // The kernels after the plan, as launchers on a stream.  Staging (a no-op
  // unless the plan staged this step) dequantises the prefill blocks; of the
  // two prefill launches of a staged call only the one the plan picked runs.
  const bool prefill_mfma = pp.mfma_prefill && max_query_len > 1;
  auto stage_on = [&](hipStream_t st) -> int {
    pkv::StageParams sp{};
    sp.cache = kv_cache_layer;
    sp.kv_scales = kv_scales;
    sp.src = pp.stage_src;
    sp.staged = wsb + stl.blocks;
    sp.hdr = hdr;
    sp.capacity = stl.capacity;
    sp.num_blocks = num_blocks;
    sp.num_kv_heads = num_kv_heads;
    sp.head_dim = head_dim;
    sp.fp8 = fp8 ? 1 : 0;
    return pkv::launch_stage(sp, std::min<int64_t>(2 * stl.capacity, (int64_t)cus * 8), st)
               ? fail(PKV_ERR_LAUNCH, "stage launch failed")
               : PKV_OK;
  };
  auto prefill_on = [&](hipStream_t ps) -> int {
    pkv::PrefillParams fp{};
    fp.out = out;
    fp.q = q;
    fp.cache = kv_cache_layer;
    fp.kv_scales = kv_scales;
    fp.kv_fp8 = fp8 ? 1 : 0;
    fp.block_table = block_table;
    fp.items = pp.prefill_items;
    fp.pf_order = pp.pf_order;
    fp.pf_slot_start = pp.pf_slot_start;
    fp.hdr = hdr;
    fp.err = hdr + pkv::kHdrError;
    fp.scale_log2 = scale_log2;
    fp.num_q_heads = num_q_heads;
    fp.num_kv_heads = num_kv_heads;
    fp.group = group;
    fp.num_blocks = num_blocks;
    fp.max_blocks_per_req = max_blocks_per_req;
    const int64_t grid = pf_per_head * num_kv_heads;
    if (stl.capacity > 0) {
      // staged: the bf16 kernel over the staged blocks (a no-op unless the
      // plan staged this step)
      pkv::PrefillParams sf = fp;
      sf.cache = wsb + stl.blocks;
      sf.kv_scales = nullptr;
      sf.kv_fp8 = 0;
      sf.block_table = pp.stage_bt;
      sf.num_blocks = (int32_t)stl.capacity;
      sf.staged = 1;
      if (pkv::launch_prefill(sf, head_dim, grid, ps)) return fail(PKV_ERR_LAUNCH, "prefill launch failed");
    }
    fp.staged = 0;
    if (pkv::launch_prefill(fp, head_dim, grid, ps)) return fail(PKV_ERR_LAUNCH, "prefill launch failed");
    return PKV_OK;
  };
  pkv::RowParams rp{};
  auto rows_and_merge = [&]() -> int {
    rp.out = out;
    rp.q = q;
    rp.cache = kv_cache_layer;
    rp.block_table = block_table;
    rp.qsl = query_start_loc;
    rp.nct = num_computed_tokens;
    rp.items = pp.row_items;
    rp.items_tail = pp.row_items_tail;
    rp.hdr = hdr;
    rp.part_o = (float*)(wsb + ws.part_o);
    rp.part_ml = (float2*)(wsb + ws.part_ml);
    rp.err = hdr + pkv::kHdrError;
    rp.scale_log2 = scale_log2;
    rp.num_q_heads = num_q_heads;
    rp.num_kv_heads = num_kv_heads;
    rp.group = group;
    const int gmax = i8 ? pkv::max_group_regs_i8(dtype) : pkv::max_group_regs(dtype, group, head_dim);
    rp.head_groups = (group + gmax - 1) / gmax;
    rp.num_blocks = num_blocks;
    rp.max_blocks_per_req = max_blocks_per_req;
    {
      const int64_t bound_waves = ws.cap_row_items * num_kv_heads * rp.head_groups;
      mark(PKV_PHASE_ROWS, 0);
      if (i8 ? pkv::launch_rows_i8(rp, kv_scales, dtype, head_dim, fp8, bound_waves, cus, s)
             : pkv::launch_rows(rp, dtype, head_dim, bound_waves, cus, s))
        return fail(PKV_ERR_LAUNCH, "row launch failed");
      mark(PKV_PHASE_ROWS, 1);
    }
    mark(PKV_PHASE_REDUCE, 0);
    if (max_seq_len > pkv::kSplitTokens) {
      pkv::ReduceParams rd{};
      rd.out = out;
      rd.items = pp.reduce_items;
      rd.hdr = hdr;
      rd.part_o = rp.part_o;
      rd.part_ml = rp.part_ml;
      rd.num_q_heads = num_q_heads;
      rd.cap_reduce = ws.cap_reduce;
      // (a workgroup per (long row, head) at most; short rows need a quarter of that)
      const int64_t bound = ws.cap_reduce * num_q_heads;
      const int64_t grid = std::min<int64_t>(bound, (int64_t)cus * 8);
      if (pkv::launch_reduce(rd, dtype, head_dim, grid, s)) return fail(PKV_ERR_LAUNCH, "reduce launch failed");
    }
    mark(PKV_PHASE_REDUCE, 1);
    return PKV_OK;
  };
  // With `overlap` (8-bit caches, no phase events) and no staging area the
  // prefill kernel (dequantising its tiles) runs on a second stream beside
  // the row kernels, which take the CUs its last workgroups leave free; the
  // caller's stream waits for it at the end (Fork).  With a staging area the
  // step runs in order on the caller's stream: the bf16 prefill beside the
  // rows measured no faster than after them (as with a bf16 cache), and the
  // staging kernel beside the FP8 row kernel slowed it.
  Fork fork;
  int rc = PKV_OK;
  mark(PKV_PHASE_PREFILL, 0);
  if (prefill_mfma && stl.capacity > 0 && (rc = stage_on(s)) != PKV_OK) return rc;
  const hipStream_t ps = prefill_mfma && overlap && stl.capacity == 0 && fork.begin(s) ? fork.side : s;
  if (prefill_mfma && (rc = prefill_on(ps)) != PKV_OK) return rc;
  mark(PKV_PHASE_PREFILL, 1);
  if ((rc = rows_and_merge()) != PKV_OK) return rc;
  if (fork.join()) return fail(PKV_ERR_LAUNCH, "joining the prefill stream failed");
  return ok();
}

int paged_attention(void* out, const void* q, const void* kv_cache_layer,
                    const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                    float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                    int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, kv_cache_layer, block_table, seq_lens, query_start_loc,
                        num_computed_tokens, scale, num_reqs, num_tokens, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, max_blocks_per_req, max_query_len, max_seq_len, dtype,
                        workspace, workspace_bytes, stream, nullptr);
}

int paged_attention_profiled(void* out, const void* q, const void* kv_cache_layer,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                             float scale, int32_t num_reqs, int64_t num_tokens,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t num_blocks, int32_t max_blocks_per_req,
                             int32_t max_query_len, int32_t max_seq_len, int32_t dtype,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* phase_events) {
  return attention_impl(out, q, kv_cache_layer, block_table, seq_lens, query_start_loc,
                        num_computed_tokens, scale, num_reqs, num_tokens, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, max_blocks_per_req, max_query_len, max_seq_len, dtype,
                        workspace, workspace_bytes, stream, phase_events);
}

}  // extern "C"

namespace {

// Device memory of paged_attention_noalloc: split-KV partials, work lists and
// the header with the error word, PKV_NOALLOC_SCRATCH_BYTES per GPU, held
// from the library's load until the process ends.  In host code the name
// `scratch` is only the runtime's handle for the array: its device address
// comes from hipGetSymbolAddress, once per device (each GPU has its own copy).
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t status = hipSuccess;
};
ScratchAddr g_scratch_addr[kMaxDevices];

// Device address of `scratch` on device `dev` (current on this thread).
void* scratch_on(int dev, hipError_t* status) {
  ScratchAddr& a = g_scratch_addr[dev];
  std::call_once(a.once, [&a] {
    void* p = nullptr;
    a.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    a.ptr = a.status == hipSuccess ? p : nullptr;
  });
  *status = a.status;
  return a.ptr;
}

// OR the step's device error word into the caller's int32.
__global__ void export_error_kernel(const int32_t* hdr, int32_t* device_error) {
  if (threadIdx.x == 0 && hdr[pkv::kHdrError] != 0) *device_error |= hdr[pkv::kHdrError];
}

}  // namespace

extern "C" {

int paged_attention_noalloc(void* out, const void* q, const void* kv_cache_layer,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                            float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                            int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                            int32_t dtype, int32_t* device_error, void* stream) {
  // the scratch this step needs, by the bound paged_attention checks its workspace against
  if (elem_bytes(dtype) == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_DIMS, "num_q_heads %lld / num_kv_heads %lld", num_q_heads, num_kv_heads);
  const size_t need = workspace_size_tiles(num_reqs, num_tokens, num_q_heads, head_dim, max_query_len,
                                           max_seq_len,
                                           tile_rows_for(dtype, head_dim, num_q_heads / num_kv_heads, false));
  if (need == 0) return fail(PKV_ERR_DIMS, "num_reqs %lld, num_tokens %lld, limits", num_reqs, num_tokens);
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE, "step needs %lld bytes of scratch; the static scratch holds %lld",
                (long long)need, (long long)PKV_NOALLOC_SCRATCH_BYTES);
  if (device_error && !aligned(device_error, 4)) return fail(PKV_ERR_ALIGN, "device_error needs 4-byte alignment");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_LAUNCH, "no usable current device (%lld)", dev);
  hipError_t st = hipSuccess;
  void* ws = scratch_on(dev, &st);
  if (ws == nullptr) return fail(PKV_ERR_LAUNCH, "hipGetSymbolAddress of the scratch failed: %lld", (long long)st);
  const int rc = attention_impl(out, q, kv_cache_layer, block_table, seq_lens, query_start_loc,
                                num_computed_tokens, scale, num_reqs, num_tokens, num_q_heads, num_kv_heads,
                                head_dim, num_blocks, max_blocks_per_req, max_query_len, max_seq_len, dtype, ws,
                                PKV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
  if (rc != PKV_OK || device_error == nullptr) return rc;
  hipLaunchKernelGGL(export_error_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const int32_t*)ws,
                     device_error);
  if (hipGetLastError() != hipSuccess) return fail(PKV_ERR_LAUNCH, "error export launch failed");
  return ok();
}

int paged_attention_int8(void* out, const void* q, const void* kv_cache_layer, const float* kv_scales,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                         float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                         int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* phase_events) {
  if (!kv_scales) return fail(PKV_ERR_NULL, "kv_scales is NULL");
  return attention_impl(out, q, kv_cache_layer, block_table, seq_lens, query_start_loc,
                        num_computed_tokens, scale, num_reqs, num_tokens, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, max_blocks_per_req, max_query_len, max_seq_len, dtype,
                        workspace, workspace_bytes, stream, phase_events, kv_scales, false, phase_events == nullptr);
}

int paged_attention_fp8(void* out, const void* q, const void* kv_cache_layer, const float* kv_scales,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                        float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                        int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                        int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                        void* const* phase_events) {
  if (!kv_scales) return fail(PKV_ERR_NULL, "kv_scales is NULL");
  return attention_impl(out, q, kv_cache_layer, block_table, seq_lens, query_start_loc,
                        num_computed_tokens, scale, num_reqs, num_tokens, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, max_blocks_per_req, max_query_len, max_seq_len, dtype,
                        workspace, workspace_bytes, stream, phase_events, kv_scales, true, phase_events == nullptr);
}

static int kv_write_8bit(const void* k, const void* v, const int64_t* slot_mapping, void* kv_cache_layer,
                         float* kv_scales, int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, int32_t* device_error, void* stream, bool fp8) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PKV_ERR_DTYPE, "dtype %lld", dtype);
  if (num_tokens < 0) return fail(PKV_ERR_DIMS, "num_tokens %lld < 0", num_tokens);
  if (num_blocks <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_DIMS, "num_blocks %lld, num_kv_heads %lld", num_blocks, num_kv_heads);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_DIMS, "head_dim %lld not 64/128", head_dim);
  if (!kv_cache_layer || !kv_scales) return fail(PKV_ERR_NULL, "kv_cache_layer or kv_scales is NULL");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v or slot_mapping is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kv_cache_layer, 16) || !aligned(kv_scales, 4) ||
      !aligned(slot_mapping, 8))
    return fail(PKV_ERR_ALIGN, "k, v, cache must be 16-byte aligned, scales 4-byte, slot_mapping 8-byte");
  if (pkv::launch_kv_write_i8(k, v, slot_mapping, kv_cache_layer, kv_scales, num_tokens, num_blocks, num_kv_heads,
                              head_dim, dtype == PKV_BF16, fp8, device_error, (hipStream_t)stream))
    return fail(PKV_ERR_LAUNCH, fp8 ? "kv_write_fp8 launch: %lld" : "kv_write_int8 launch: %lld",
                (long long)hipGetLastError());
  return ok();
}

int paged_kv_write_int8(const void* k, const void* v, const int64_t* slot_mapping, void* kv_cache_layer,
                        float* kv_scales, int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, int32_t dtype, int32_t* device_error, void* stream) {
  return kv_write_8bit(k, v, slot_mapping, kv_cache_layer, kv_scales, num_tokens, num_blocks, num_kv_heads,
                       head_dim, dtype, device_error, stream, false);
}

int paged_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* kv_cache_layer,
                       float* kv_scales, int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t dtype, int32_t* device_error, void* stream) {
  return kv_write_8bit(k, v, slot_mapping, kv_cache_layer, kv_scales, num_tokens, num_blocks, num_kv_heads,
                       head_dim, dtype, device_error, stream, true);
}

int32_t pkv_read_device_error(const void* workspace, void* stream) {
  if (!workspace) return -1;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return -1;
  int32_t e = 0;
  if (hipMemcpy(&e, workspace, sizeof(e), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return e;
}

int pkv_validate_metadata_host(const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* query_start_loc,
                               const int32_t* num_computed_tokens, const int64_t* slot_mapping,
                               int32_t num_reqs, int64_t num_tokens, int32_t num_blocks,
                               int32_t max_blocks_per_req, int32_t max_query_len,
                               int32_t max_seq_len) {
  if (num_reqs < 0 || num_tokens < 0 || num_blocks <= 0 || max_blocks_per_req <= 0)
    return fail(PKV_ERR_DIMS, "num_reqs %lld, num_tokens %lld, num_blocks %lld", num_reqs,
                num_tokens, num_blocks);
  if (!query_start_loc) return fail(PKV_ERR_NULL, "query_start_loc is NULL");
  if (num_reqs > 0 && (!block_table || !seq_lens || !num_computed_tokens))
    return fail(PKV_ERR_NULL, "block_table, seq_lens or num_computed_tokens is NULL");
  if (query_start_loc[0] != 0) return fail(PKV_ERR_METADATA, "query_start_loc[0] = %lld", query_start_loc[0]);
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int64_t qs = query_start_loc[r], qe = query_start_loc[r + 1];
    const int64_t ql = qe - qs, L = seq_lens[r], c = num_computed_tokens[r];
    if (ql < 0 || qe > num_tokens)
      return fail(PKV_ERR_METADATA, "request %lld: query_start_loc %lld..%lld", r, qs, qe);
    if (c < 0 || L != c + ql)
      return fail(PKV_ERR_METADATA, "request %lld: seq_len %lld != computed + query_len (%lld)", r, L,
                  c + ql);
    if (ql > max_query_len || L > max_seq_len || L > (int64_t)max_blocks_per_req * pkv::kBlock)
      return fail(PKV_ERR_METADATA, "request %lld: query_len %lld / seq_len %lld over the limits", r,
                  ql, L);
    const int64_t nb = (L + pkv::kBlock - 1) / pkv::kBlock;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = block_table[(int64_t)r * max_blocks_per_req + j];
      if (b < 0 || b >= num_blocks)
        return fail(PKV_ERR_METADATA, "request %lld: block_table[%lld] = %lld out of range", r, j, b);
    }
  }
  if (slot_mapping) {
    std::vector<int64_t> used;
    used.reserve((size_t)num_tokens);
    for (int64_t t = 0; t < num_tokens; ++t) {
      const int64_t s = slot_mapping[t];
      if (s == -1) continue;
      if (s < 0 || s >= (int64_t)num_blocks * pkv::kBlock)
        return fail(PKV_ERR_METADATA, "token %lld: slot %lld outside the pool", t, s);
      used.push_back(s);
    }
    std::sort(used.begin(), used.end());
    for (size_t i = 1; i < used.size(); ++i)
      if (used[i] == used[i - 1]) return fail(PKV_ERR_METADATA, "slot %lld used twice", used[i]);
  }
  return ok();
}

}  // extern "C"
