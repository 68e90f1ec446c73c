// Device-side helpers and the workspace layout shared by the kernels and the
// host entry points of libpagedkv (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;        // tokens per cache block (fixed)
constexpr int kWave = 64;         // CDNA wavefront width
// Split-KV partition length of a decode row: a constant, so a row's result
// never depends on the rest of the batch.  Each partition is one work item of
// a row kernel; 1024 tokens measured 4-8% faster row kernels than 512 on the
// mixed, GQA and long-context decodes (bf16 and 8-bit caches alike: fewer,
// longer items, fewer partials to write and merge) and unchanged or faster
// on the Llama-7B-shaped one.
constexpr int kSplitTokens = 1024;
constexpr int kSplitBlocks = kSplitTokens / kBlock;
constexpr int kMaxGroupRegs = 4;  // query heads per kv head handled by one wave

// Header words at the start of the workspace (int32).
enum HdrWord {
  kHdrError = 0,
  kHdrRowItems = 1,
  kHdrPrefillItems = 2,
  kHdrReduceItems = 3,
  kHdrSlots = 4,
  kHdrRowHead = 5,      // row items in the first region (the rest are in the tail region)
  kHdrPrefillStatic = 6,  // 1: prefill items come from per-slot lists (pf_order), 0: from the queues
  kHdrReduceShort = 7,  // reduce items of short rows, listed first (the rest fill the list from its end)
  kHdrReduceSplit = 8,  // of the rest, rows of more than 2 * PlanParams::reduce_short_parts partitions
  kHdrPrefillStaged = 9,   // 1: the prefill reads bf16 blocks dequantised once into the staging area
  kHdrStagedBlocks = 10,   // blocks in the staging area this step (0 when not staged)
  kHdrPrefillQueue = 16,  // one prefill work-queue counter per kv head (zeroed by the plan kernel)
};
constexpr int kMaxKvHeads = 240;  // kv heads with a prefill queue counter in the header
constexpr int kPfMaxSlots = 64;   // static prefill assignment: at most this many workgroups per kv head
constexpr int kPfMaxStatic = 256; // ... and at most this many prefill items
constexpr size_t kHdrBytes = 1024;
static_assert((kHdrPrefillQueue + kMaxKvHeads) * 4 <= kHdrBytes, "header too small");

// Reduce item (int4): x = query row, y = request, z = partitions, w = first
// partial slot.  Rows of at most PlanParams::reduce_short_parts partitions
// are listed from the front of the list, longer rows from its end (position
// cap - 1 - i), so the merge can batch the short ones.

// Row item (int4): x = query row, y = request, z = partition (kWholeRow: all
// visible keys, kNanRow: metadata was bad, write NaN), w = first partial slot
// of the row (or -1 when the item writes `out` directly).
constexpr int kWholeRow = -1;
constexpr int kNanRow = -2;

// Prefill item (int4): x = request, y = the tile's first query token (its
// row of q and out), z = rows in the tile, w = num_computed_tokens minus the
// request's first query token, so y + w is the tile's first position.  The
// prefill kernel needs no other per-request metadata than the block table.

struct WsLayout {
  size_t row_items, row_items_tail, prefill_items, reduce_items, pf_order, pf_slot_start, part_ml, part_o, total;
  int64_t cap_row_items, cap_prefill_items, cap_reduce, cap_slots;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Staging area of an 8-bit cache's prefill: the workspace bytes past
// WsLayout::total.  A bf16 block table of the same shape as the step's
// ([num_reqs][max_blocks_per_req] int32), the source block of each staged
// block (int32 [capacity]), then the staged blocks, laid out as a bf16 cache
// of `capacity` blocks ([2][capacity][16][num_kv_heads][head_dim]).
struct StageLayout {
  size_t bt, src, blocks;   // byte offsets from the workspace start
  int64_t capacity;         // staged blocks that fit (0: no staging)
};
inline int64_t stage_block_bytes(int64_t num_kv_heads, int64_t head_dim) {
  return 2 * 16 * num_kv_heads * head_dim * 2;   // K and V halves of one block, bf16
}
inline StageLayout stage_layout(size_t ws_total, size_t workspace_bytes, int64_t num_reqs,
                                int64_t max_blocks_per_req, int64_t num_kv_heads, int64_t head_dim) {
  StageLayout s{};
  s.bt = align_up(ws_total, 256);
  s.src = align_up(s.bt + sizeof(int32_t) * (size_t)(num_reqs * max_blocks_per_req), 256);
  if (workspace_bytes <= s.src + 512) return s;
  const int64_t per = stage_block_bytes(num_kv_heads, head_dim) + (int64_t)sizeof(int32_t);
  int64_t cap = (int64_t)(workspace_bytes - s.src - 512) / per;
  if (cap > ((int64_t)1 << 30)) cap = (int64_t)1 << 30;
  s.blocks = align_up(s.src + sizeof(int32_t) * (size_t)cap, 256);
  while (cap > 0 && s.blocks + (size_t)cap * (size_t)stage_block_bytes(num_kv_heads, head_dim) > workspace_bytes) {
    --cap;
    s.blocks = align_up(s.src + sizeof(int32_t) * (size_t)cap, 256);
  }
  s.capacity = cap;
  return s;
}

// Capacities are upper bounds that hold for any metadata that passes the
// device checks (query_len <= max_query_len, seq_len <= max_seq_len).
inline WsLayout ws_layout(int64_t num_reqs, int64_t num_tokens, int64_t num_q_heads,
                          int64_t head_dim, int64_t max_query_len, int64_t max_seq_len,
                          int64_t prefill_tile_rows) {
  WsLayout w{};
  const int64_t dec_rows = num_reqs < num_tokens ? num_reqs : num_tokens;
  const int64_t max_parts = (max_seq_len + kSplitTokens - 1) / kSplitTokens;
  w.cap_row_items = dec_rows * (max_parts > 1 ? max_parts : 1) + num_tokens + 1;
  w.cap_prefill_items = num_tokens / (prefill_tile_rows > 0 ? prefill_tile_rows : 1) + num_reqs + 1;
  w.cap_reduce = dec_rows + 1;
  w.cap_slots = (max_parts > 1 ? dec_rows * max_parts : 0) + 1;
  (void)max_query_len;
  size_t off = kHdrBytes;
  w.row_items = off;      off = align_up(off + sizeof(int32_t) * 4 * w.cap_row_items, 256);
  w.row_items_tail = off; off = align_up(off + sizeof(int32_t) * 4 * w.cap_row_items, 256);
  w.prefill_items = off;  off = align_up(off + sizeof(int32_t) * 4 * w.cap_prefill_items, 256);
  w.reduce_items = off;   off = align_up(off + sizeof(int32_t) * 4 * w.cap_reduce, 256);
  w.pf_order = off;       off = align_up(off + sizeof(int32_t) * kPfMaxStatic, 256);
  w.pf_slot_start = off;  off = align_up(off + sizeof(int32_t) * (kPfMaxSlots + 1), 256);
  w.part_ml = off;        off = align_up(off + sizeof(float) * 2 * w.cap_slots * num_q_heads, 256);
  w.part_o = off;         off = align_up(off + sizeof(float) * w.cap_slots * num_q_heads * head_dim, 256);
  w.total = off;
  return w;
}

#ifdef __HIP_DEVICE_COMPILE__
#define PKV_DEV __device__ __forceinline__
#else
#define PKV_DEV __device__ inline
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 is stored as its 16-bit pattern; a bf16 value is the top half of the
// float32 with the same value.
PKV_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
PKV_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even, NaN stays NaN (v_cvt_pk_bf16_f32).
PKV_DEV uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// a.lo*b.lo + a.hi*b.hi + c, bf16 products accumulated in fp32.
PKV_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane moves (all rows and banks enabled).
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;   // rotate right by 4 inside each row of 16 lanes
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
PKV_DEV float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

PKV_DEV float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

PKV_DEV float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

PKV_DEV float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// max / sum of x[l] and x[l ^ 16], and of x[l] and x[l ^ 32], for every lane l
// (v_permlane16_swap / v_permlane32_swap: VALU, no LDS round trip).
PKV_DEV float xmax16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
PKV_DEV float xmax32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
PKV_DEV float xsum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
PKV_DEV float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The 4 OCP E4M3 codes of w (byte order) as float (v_cvt_pk_f32_fp8: every
// E4M3 value is a float32 value, so the conversion is exact).
PKV_DEV void fp8x4(uint32_t w, float (&f)[4]) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource over [p, p + bytes); loads past the end return 0.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (NT).  The decode
// kernels read V with it: measured on the decode workloads, it raises the
// row kernels' stream rate by 2-12% (K and V both non-temporal is slower
// than V alone, and so is K alone on most of them).
constexpr int kCpolNT = 2;
// Read of step metadata (work items, query_start_loc, num_computed_tokens)
// through the constant address space.  At a wave-uniform index it compiles to
// a scalar load, whose completion is tracked by its own counter: waiting for
// it does not also wait for the vector loads of the cache stream and the
// output stores in flight, as a vector load's wait would.  Only for arrays no
// kernel writes while the reading kernel runs.
PKV_DEV int load_const(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
PKV_DEV int4 load_const(const int4* p, int64_t i) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  const i32x4_t x = ((const __attribute__((address_space(4))) i32x4_t*)p)[i];
  return make_int4(x.x, x.y, x.z, x.w);
}

PKV_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

}  // namespace pkv
