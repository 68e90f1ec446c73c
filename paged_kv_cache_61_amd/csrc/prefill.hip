// Causal chunked prefill over the paged cache on bf16 MFMA (gfx950).
//
// What is computed ("AI Infra入门干货总结：大模型是如何高效推理的", sections
// "Paged Attention" and "LLM 推理全流程" / "Attention (FlashAttention)"; the
// definition is softmax(q k^T * scale + mask) v, lpnh.cn/news/2669538 2.1):
// a prefill chunk of request r covers query rows i = 0 .. query_len-1 at
// absolute positions c + i (c = num_computed_tokens); row i attends to keys
// 0 .. c + i, i.e. the whole cached prefix plus the chunk causally (chunked
// prefill: lpnh.cn/news/2436702 section 2.3).  Key t is read from physical
// block block_table[r][t / 16], offset t % 16.  Prefill is a dense
// contraction (same page, "Prefill vs Decode": compute bound), so both
// products run on the matrix cores; the score and probability matrices never
// leave the chip (tiling + online softmax, section "FlashAttention 核心").
//
// Work item = (request, tile of BQ query positions, kv head g).  The G query
// heads of group g share every K/V tile (GQA by index mapping): the tile's
// 256 MFMA rows are (position, head) pairs, position-major, BQ = 256 / G.
//
// Per 64-key tile, each of the 8 waves owns 32 rows and computes
//   S^T = K Q^T      (v_mfma_f32_32x32x16_bf16: A = K from LDS, B = Q from
//                     registers), so lane l holds the scores of row l % 32;
//   online softmax   per lane: the row max needs one exchange with lane l^32
//                     (the other 32 keys of the tile; v_permlane32_swap, no
//                     LDS round trip); exp2 with scale*log2 e
//                     folded in; rescaling skipped when no row max moved;
//   O^T += V^T P^T   (A = V^T from LDS, B = P from the S^T registers packed
//                     to bf16), so O's rows are again lane-local.
// Tiles of 64 keys stream from the cache into a 4-slot LDS ring with
// buffer_load ... lds (no staging registers): each wave copies one cache
// block (16 token rows) of K (waves 0-3) or V (waves 4-7), two tiles ahead of
// the tile being computed; the buffer descriptor of a block covers only the
// rows before the chunk's last key, so later rows read as zeros and tail
// garbage or NaN in the cache never reaches the output.  Rows are stored as
// they are in the cache (256 bytes for head_dim 128) with 16-byte chunk c of
// row r at position c ^ swz(r mod 16), swz = the two 2-bit halves of r
// swapped.  The LDS serves 256 bytes (all 64 banks) per clock: 16 lanes of a
// 16-byte read or 32 lanes of an 8-byte one.  swz is a permutation, so the K
// operand reads (16 consecutive keys, one chunk) hit 16 distinct positions;
// and its upper two bits differ within each aligned group of 4 rows, so a
// transposed V read (32 lanes: 4 rows x 4 adjacent chunks of an aligned
// group of 4) also hits 16 distinct positions.  Neither read conflicts on
// banks.  (A swizzle that only keeps 16-lane halves apart, or a plain
// c ^ (r mod 16), makes the transposed reads conflict two or four ways.)  The
// V^T operand of the second product comes from ds_read_b64_tr_b16 (two 4-key
// transposed reads per lane), in the key order of the S^T accumulator
// (8*(i/4) + 4*(l/32) + i%4).
// The two waves on each SIMD alternate ("ping-pong"): while one issues the
// MFMAs of a tile (PV of the previous tile, QK of this one) the other runs
// its softmax; one workgroup barrier per tile starts the two groups half a
// tile apart (see the schedule in the kernel).
// Causal masks are applied only on tiles that cross a row's position.
#include <math.h>

#include <type_traits>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfRows = 256;   // MFMA rows per workgroup (8 waves x 32)
constexpr int kPfKeys = 64;    // keys per tile (4 cache blocks)
constexpr int kPfThreads = 512;
constexpr int kStages = 4;     // ring slots: tiles t-1 (PV), t (QK), t+1 and t+2 (in flight)

// Sizes that follow from head_dim (64 or 128).
template <int D>
struct PfCfg {
  static constexpr int kRowB = D * 2;               // bytes of one key row (one kv head)
  static constexpr int kHalfTile = kPfKeys * kRowB; // K or V part of a tile: 8 or 16 KiB
  static constexpr int kStage = 2 * kHalfTile;      // one ring slot: K then V
  static constexpr int kKSteps = D / 16;            // Q.K k-steps
  static constexpr int kDTiles = D / 32;            // O^T row tiles
  static constexpr int kCopyLoads = kBlock * kRowB / 1024;  // 16-byte-per-lane loads per cache block
};
constexpr int kD = 128;        // head_dim of the 8-bit cache instantiations
// 8-bit cache (INT8 or FP8 E4M3 codes): the copies bring codes (128-byte
// rows) and per-row scales into a 4-slot ring, three tiles ahead; every
// period the waves dequantise K(t+1) and V(t) (value * scale in float32,
// rounded to bf16) into two K and two V tiles laid out like the bf16 ring's
// halves, which the MFMA phases read.
constexpr int kRowB8 = kD;                        // bytes of one int8 key row
constexpr int kHalf8 = kPfKeys * kRowB8;          // codes of K or V of a tile: 8 KiB
constexpr int kScl = kPfKeys * 4;                 // scales of K or V of a tile
constexpr int kStage8 = 2 * kHalf8 + 2 * kScl;    // one int8 ring slot
constexpr int kStages8 = 4;
constexpr int kConv = kStages8 * kStage8;         // offset of the bf16 tiles K0, K1, V0, V1
constexpr int kLdsI8 = kConv + 4 * PfCfg<kD>::kHalfTile;
static_assert(kLdsI8 + 64 <= 160 * 1024, "8-bit prefill LDS");

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define PKV_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define PKV_INLINE __attribute__((always_inline))

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class Fn>
PKV_DEV void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

PKV_DEV f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Pack two fp32 to a bf16 pair (round to nearest even, v_cvt_pk_bf16_f32),
// low element first.
PKV_DEV uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// max(x[l], x[l ^ 32]) for every lane l.  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second (a VALU
// op, no LDS round trip): with x in both, one result holds each lane's own
// value and the other its partner's.
PKV_DEV float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x[l] + x[l ^ 32] for every lane l (v_permlane32_swap, as in pair_max).
PKV_DEV float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A row's reference max moves only when a tile's max exceeds it by more than
// this (log2 units); p = exp2(s - ref) stays <= 2^8 and O is rescaled rarely.
constexpr float kRefSlack = 8.f;

// Chunk-position permutation of key row r (mod 16) inside a K or V tile:
// 16-byte chunk c of the row sits at position c ^ swz<D>(r), so both the K
// operand reads and the transposed V reads are free of bank conflicts.
//  * D = 128 (256-byte rows, 16 chunks; every row starts at bank 0): swz
//    swaps the two 2-bit halves of r.  It is a permutation of 0..15, so 16
//    rows read at one chunk hit 16 distinct positions; and its upper two
//    bits differ within each aligned group of 4 rows, so a transposed read
//    (4 rows x 4 adjacent chunks) covers 16 distinct positions too.
//  * D = 64 (128-byte rows, 8 chunks; odd rows start at the upper half of
//    the banks): swz = 4 * bit1(r) + (r >> 2) mod 4.  Over the 8 even rows
//    of 16 (and over the 8 odd ones) it takes every value 0..7, so 16 rows
//    at one chunk hit 16 distinct positions; rows 4a and 4a + 2 (and 4a + 1,
//    4a + 3) differ in bit 2, so the two rows of a bank half in a transposed
//    read put an aligned group of 4 chunks on complementary positions.
template <int D>
PKV_DEV int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r & 2) << 1) | ((r >> 2) & 3);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (expcnt and lgkmcnt left alone).
template <int N>
PKV_DEV void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for this wave's global stores to complete.
PKV_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One cache block into LDS: four buffer_load_dwordx4 ... lds, instruction j
// copying 16 bytes per lane at voff[j] inside the buffer described by `rs`
// (zeros past its end) to LDS byte offset m0v + 1024 j + 16 * lane (m0v
// wave-uniform).  Inline asm, so the compiler does not order its own LDS
// reads behind these loads (completion is awaited explicitly with wait_vmem
// before the barrier that publishes a tile).  The compiler does not insert
// hazard waits inside inline asm, so the asm carries its own: the descriptor
// words may have been written by VALU instructions (readfirstlane), which a
// vector memory instruction may read only five wait states later (the leading
// s_nop 4, which also covers the compiler's M0 write), and an M0 write needs
// one wait state before an LDS-DMA instruction uses it.
PKV_DEV void dma_block(const u32x4& rs, const uint32_t (&voff)[4], uint32_t m0v) {
  // M0 is an in/out operand: the compiler loads it before the asm and knows
  // the asm leaves it stepped by 3 KiB.
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen lds"
      : "+{m0}"(m0v)
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rs)
      : "memory", "scc");
}

// Two buffer_load_dwordx4 ... lds (LDS offsets m0v and m0v + 1 KiB), with
// the same hazard waits as dma_block.
PKV_DEV void dma_pair(const u32x4& rs, uint32_t v0, uint32_t v1, uint32_t m0v) {
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds"
      : "+{m0}"(m0v)
      : "v"(v0), "v"(v1), "s"(rs)
      : "memory", "scc");
}
// buffer_load_dword ... lds: each active lane copies 4 bytes at voff to LDS
// offset m0v + 4 * lane.
PKV_DEV void dma_dword(const u32x4& rs, uint32_t voff, uint32_t m0v) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds" : "+{m0}"(m0v) : "v"(voff), "s"(rs) : "memory");
}


// Descriptor words for raw (stride 0) buffer access to [base, base + bytes).
PKV_DEV u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), (uint32_t)kRsrcWord3};
}

// The metadata arrays are passed on their own as restrict pointers so their
// wave-uniform reads become scalar loads, which never wait on the tile stream.
template <int D, bool I8, bool FP8>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(
    PrefillParams a, const int4* __restrict__ items, const int32_t* __restrict__ block_table) {
  static_assert(D == 128 || (D == 64 && !I8), "bf16 cache: head_dim 64 or 128; 8-bit cache: 128");
  using Cf = PfCfg<D>;
  constexpr int kRowB = Cf::kRowB, kHalfTile = Cf::kHalfTile, kStage = Cf::kStage;
  constexpr int kKSteps = Cf::kKSteps, kDTiles = Cf::kDTiles;
  __shared__ __attribute__((aligned(16))) char lds[I8 ? kLdsI8 : kStages * kStage];
  __shared__ int tile_bad[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index, made visibly wave-uniform so everything derived from it is scalar
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;        // which 8-wide k group of the MFMA operand
  const int lrow = lane & 31;        // MFMA row / column owned by the lane
  const int G = a.group;
  const int BQ = kPfRows / G;        // query positions per tile
  const int Hkv = a.num_kv_heads;
  const size_t row_bytes = (size_t)Hkv * (I8 ? kRowB8 : kRowB);  // bytes between token rows
  const size_t blk_bytes = kBlock * row_bytes;
  const char* kbase = (const char*)a.cache;
  const char* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  const float sl2 = a.scale_log2;
  const float csc = fabsf(sl2);

  // Copy role: wave w streams block (w & 3) of each tile, of K (w < 4) or V.
  const int cblk = w & 3;
  const char* cbase = w < 4 ? kbase : vbase;
  const int ldst_half = I8 ? (w < 4 ? 0 : kHalf8) + cblk * kBlock * kRowB8 : (w < 4 ? 0 : kHalfTile) + cblk * kBlock * kRowB;

  // V^T transpose-read geometry (per lane, independent of the tile).
  const int ts = lane & 15;                            // source lane inside a 16-lane group
  const int tdb = ((lane >> 4) & 1) * 16 + 4 * (ts & 3);  // head_dim offset inside a 32-wide tile

  // Persistent grid over query tiles listed longest first.  Workgroup b keeps
  // kv head b mod Hkv; with 8 kv heads and a grid that is a multiple of 8,
  // workgroup b runs on XCD b mod 8, so an XCD's L2 serves one head's K/V to
  // all of its query tiles.  The workgroups of a head take the head's tiles
  // from a queue (an atomic counter that the plan kernel zeroes) in list
  // order, each as soon as it is free, so the longest tiles are spread first
  // and the work per workgroup evens out.  The next index is fetched while
  // the current tile runs.
  // An 8-bit cache's step launches this kernel twice, over the staging area
  // (bf16, staged = 1) and over the cache (staged = 0); the plan's decision
  // picks the one that runs.
  if (a.hdr[kHdrPrefillStaged] != a.staged) return;
  const int n_entries = a.hdr[kHdrPrefillItems];
  const int g = blockIdx.x % Hkv;
  // (8-bit cache) scales [2][num_blocks][Hkv][16] fp32: this wave's K or V
  // half, and inside a block the 16 contiguous scales of kv head g
  const float* sbase = a.kv_scales + (w < 4 ? 0 : (size_t)a.num_blocks * kBlock * Hkv) + (size_t)g * kBlock;

  // Copy geometry, the same for every tile: instruction j, lane L of this
  // wave's block copy carries token row 4j + L/16 of the block and the chunk
  // that lands at LDS position L mod 16 (chunk (L mod 16) ^ swz(row)); the
  // destination is this wave's quarter of a ring slot's K or V half.
  // (8-bit cache: instruction j < 2 fills LDS rows s = 8j + L/8 of the block, 16
  // codes of token row s ^ bit2(s) each, so rows r and r + 4 sit in opposite
  // bank halves for the dequantisation reads; voff[2] is the scale of token
  // row L of the block, L < 16, among kv head g's 16 contiguous scales.)
  uint32_t voff[4];
  if constexpr (I8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sr = 8 * j + (lane >> 3);      // LDS row inside the block
      const int tr = sr ^ ((sr >> 2) & 1);     // token row it holds
      voff[j] = tr * (uint32_t)row_bytes + g * kRowB8 + ((lane & 7) << 4);
    }
    voff[2] = (uint32_t)(lane & 15) * 4u;
    voff[3] = 0;
  } else {
    // 16 lanes per row of 256 bytes (D = 128) or 8 per row of 128 bytes (D = 64)
    constexpr int kLanesPerRow = kRowB / 16;
#pragma unroll
    for (int j = 0; j < Cf::kCopyLoads; ++j) {
      const int rb = (64 / kLanesPerRow) * j + lane / kLanesPerRow;
      voff[j] = rb * (uint32_t)row_bytes + g * kRowB + (((lane % kLanesPerRow) ^ swz<D>(rb)) << 4);
    }
#pragma unroll
    for (int j = Cf::kCopyLoads; j < 4; ++j) voff[j] = 0;
  }
  const uint32_t ldst = (uint32_t)(uintptr_t)PKV_LDS(lds) + (uint32_t)ldst_half;
  const uint32_t ldsc = (uint32_t)(uintptr_t)PKV_LDS(lds) + (uint32_t)(2 * kHalf8 + (w < 4 ? 0 : kScl) + cblk * kBlock * 4);
  const uint32_t blk_bytes32 = (uint32_t)blk_bytes;
  int* queue = a.hdr + kHdrPrefillQueue + g;
  // Items come either from the plan's static assignment (this workgroup's
  // slot blockIdx.x / Hkv: a list in pf_order, the same for every head) or,
  // when the plan did not build one, from the head's queue.
  const bool from_list = a.hdr[kHdrPrefillStatic] != 0;
  int list_pos = 0, list_base = 0, list_len = 0;
  if (from_list) {
    const int slot = blockIdx.x / Hkv;
    list_base = a.pf_slot_start[slot];
    list_len = a.pf_slot_start[slot + 1] - list_base;
  }
  auto take = [&]() PKV_INLINE -> int {   // the next item index (thread 0 only)
    if (!from_list) return atomicAdd(queue, 1);
    const int e = list_pos < list_len ? a.pf_order[list_base + list_pos++] : n_entries;
    return (unsigned)e < (unsigned)n_entries ? e : n_entries;
  };
  __shared__ int next_item[2];
  if (tid == 0) next_item[0] = take();
  __syncthreads();

  // State of the item being run, set by begin_item.
  int r = 0, tpos0 = 0, nrows = 0, kv_end = 0, ntiles = 0, pos_abs = 0, nxt = 0;
  const int32_t* bt = block_table;
  int ids0 = 0, ids1 = 0;   // block ids, see begin_item
  bool bad = false, row_ok = false;
  size_t qrow = 0;
  u32x4 qf[kKSteps];
  const int rho = w * 32 + lrow;  // this lane's MFMA row inside a tile
  // With a negative scale, q's sign is flipped (exact in bf16) and |scale|
  // used, so the row max of the raw dots is the max of the scaled scores.
  const uint32_t qsign = sl2 < 0.f ? 0x80008000u : 0u;

  // Stream tile `tile` into ring slot tile % kStages: this wave's block,
  // 4 instructions of 4 token rows; lane L of instruction j carries chunk
  // (L & 15) ^ row of token row 4j + L/16, so LDS holds the swizzled layout.
  // Straight-line: the id comes from a lane of ids0 / ids1 (blocks past
  // kv_end hold id 0 and get a zero-length buffer, which reads as zeros).
  auto issue_tile = [&](int tile) PKV_INLINE {
    const int nvalid = kv_end - (tile * kPfKeys + kBlock * cblk);  // rows of this block before kv_end
    const uint32_t nbytes = (uint32_t)min(max(nvalid, 0), kBlock) * (uint32_t)row_bytes;
    uint32_t phys;
    if (tile < 128) {
      const uint32_t p0 = (uint32_t)__builtin_amdgcn_readlane(ids0, tile & 63);
      const uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane(ids1, tile & 63);
      phys = tile < 64 ? p0 : p1;
    } else {  // items longer than 8192 keys: the table is read here
      int p = nvalid > 0 ? bt[tile * (kPfKeys / kBlock) + cblk] : 0;
      if (p < 0 || p >= a.num_blocks) {
        bad = true;
        p = 0;
      }
      phys = (uint32_t)p;
    }
    const u32x4 rs = buffer_desc(cbase + (uint64_t)phys * blk_bytes32, nbytes);
    if constexpr (I8) {
      // codes (2 instructions) and scales (1): three vector-memory operations per tile
      const uint32_t sbytes = (uint32_t)min(max(nvalid, 0), kBlock) * 4u;
      const u32x4 rss = buffer_desc(sbase + (size_t)phys * kBlock * Hkv, sbytes);
      const uint32_t slot = (uint32_t)(tile & (kStages8 - 1)) * kStage8;
      static_assert(8 * kRowB8 == 0x400, "dma_pair steps M0 by 1 KiB (8 token rows)");
      dma_pair(rs, voff[0], voff[1], ldst + slot);
      if (lane < kBlock) dma_dword(rss, voff[2], ldsc + slot);
    } else {
      const uint32_t m0 = ldst + (uint32_t)(tile & (kStages - 1)) * kStage;
      if constexpr (D == 128) {
        static_assert(4 * Cf::kRowB == 0x400, "dma_block steps M0 by 1 KiB (4 token rows)");
        dma_block(rs, voff, m0);
      } else {
        static_assert(8 * Cf::kRowB == 0x400, "dma_pair steps M0 by 1 KiB (8 token rows)");
        dma_pair(rs, voff[0], voff[1], m0);
      }
    }
  };

  // Start item ee: thread 0 takes the next queue index (published when this
  // item starts running), then the descriptor, this wave's block ids for
  // tiles 0..127 (tile l in lane l of ids0, tile 64 + l in ids1; block
  // 4*tile + cblk is read only when it holds keys before kv_end; ids outside
  // the pool are reported once per item and replaced by block 0, so the tile
  // stream never copies from outside the cache), the q rows (loads left in
  // flight) and the copies of the first two tiles.  For every item but the
  // first this runs right after the previous item's tile loop, so these
  // latencies overlap that item's epilogue.
  auto begin_item = [&](int ee) PKV_INLINE {
    if (tid == 0) nxt = take();
    const int4 item = items[ee];   // the one metadata read before the block ids
    r = item.x;
    const int tok0 = item.y;      // the tile's first query token
    nrows = item.z;
    tpos0 = (int)((int64_t)item.y + item.w);  // its position: num_computed_tokens + first row
    kv_end = tpos0 + nrows;       // keys 0 .. kv_end-1 are read
    ntiles = (kv_end + kPfKeys - 1) / kPfKeys;
    bt = block_table + (size_t)r * a.max_blocks_per_req;
    const int kb0 = (kPfKeys / kBlock) * lane + cblk;
    const int kb1 = kb0 + 64 * (kPfKeys / kBlock);
    int i0 = kBlock * kb0 < kv_end ? bt[kb0] : 0;
    int i1 = kBlock * kb1 < kv_end ? bt[kb1] : 0;
    int pos = rho / G;
    const int head = rho - pos * G;
    row_ok = rho < BQ * G && pos < nrows;
    if (!row_ok) pos = nrows - 1;  // padding rows: any visible row, loaded and zeroed
    pos_abs = tpos0 + pos;
    qrow = ((size_t)(tok0 + pos) * a.num_q_heads + g * G + head) * D;
    const uint32_t qmask = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qf[ks] = (*(const u32x4*)((const uint16_t*)a.q + qrow + ks * 16 + 8 * half) ^ qsign) & qmask;
    const bool bad0 = i0 < 0 || i0 >= a.num_blocks, bad1 = i1 < 0 || i1 >= a.num_blocks;
    bad = __any(bad0 || bad1);
    ids0 = bad0 ? 0 : i0;
    ids1 = bad1 ? 0 : i1;
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    if (I8 && ntiles > 2) issue_tile(2);
  };

  // (8-bit cache) Dequantisation role: lane L = 16a + 8b + k of wave w handles
  // tile row r = 8w + 4b + a, codes 16k .. 16k+15 (LDS row r ^ b of the int8
  // slot), and writes them as bf16 chunks 2k and 2k+1 of row r at their
  // swizzled positions; each 16-lane group covers rows of opposite bank
  // halves (reads) and opposite chunk parity (writes), so neither conflicts.
  const int cv_r = 8 * w + 4 * ((lane >> 3) & 1) + (lane >> 4);
  const int cv_rd = (cv_r ^ ((lane >> 3) & 1)) * kRowB8 + (lane & 7) * 16;
  const int cv_w0 = cv_r * kRowB + (((2 * (lane & 7)) ^ swz<D>(cv_r & 15)) << 4);
  const int cv_w1 = cv_r * kRowB + (((2 * (lane & 7) + 1) ^ swz<D>(cv_r & 15)) << 4);
  auto dequant = [&](int tile, int kv) PKV_INLINE {  // kv 0: K, 1: V
    const char* slot = lds + (tile & (kStages8 - 1)) * kStage8;
    const u32x4 cw = *(const u32x4*)(slot + kv * kHalf8 + cv_rd);
    const float sc = *(const float*)(slot + 2 * kHalf8 + kv * kScl + cv_r * 4);
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if constexpr (FP8) {
        float f[4];
        fp8x4(cw[d], f);
        o[2 * d] = pack_bf16(f[0] * sc, f[1] * sc);
        o[2 * d + 1] = pack_bf16(f[2] * sc, f[3] * sc);
      } else {
        const int x = (int)cw[d];
        o[2 * d] = pack_bf16((float)((x << 24) >> 24) * sc, (float)((x << 16) >> 24) * sc);
        o[2 * d + 1] = pack_bf16((float)((x << 8) >> 24) * sc, (float)(x >> 24) * sc);
      }
    }
    char* dst = lds + kConv + (2 * kv + (tile & 1)) * kHalfTile;
    *(u32x4*)(dst + cv_w0) = u32x4{o[0], o[1], o[2], o[3]};
    *(u32x4*)(dst + cv_w1) = u32x4{o[4], o[5], o[6], o[7]};
  };

  int e = next_item[0];
  if (e < n_entries) begin_item(e);
  for (int par = 1; e < n_entries; par ^= 1) {
    wait_vmem<0>();  // q and the first tiles are in (and earlier stores done)
    if (tid == 0) {
      next_item[par] = nxt;
      tile_bad[par] = 0;
    }
    if constexpr (I8) {  // K(0) is needed in period 0
      __builtin_amdgcn_s_barrier();
      dequant(0, 0);
    }

    f32x16 oacc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Ping-pong over two wave groups, waves 0-3 and 4-7 (every SIMD runs one
    // wave of each).  A tile's work is cut into an MFMA phase,
    //   mfma(t): O^T += V(t-1)^T P(t-1) (t >= 1), then S^T(t) = K(t) Q^T (t < n),
    // and a VALU phase,
    //   vec(t):  causal mask, online softmax of S(t) -> P(t) (and the rare O
    //            rescale, after PV(t-1) and before PV(t)).
    // A workgroup barrier starts every tile period; in period t group 0 runs
    // mfma(t) then vec(t), group 1 vec(t-1) then mfma(t), so on every SIMD one
    // wave starts the period with its MFMAs while the other runs its softmax.
    // Inside a period the two waves are not synchronised again (a barrier
    // between the phases costs more than the alternation it enforces).  Tile
    // u must be in LDS from period u on: every wave issues its copies of it in
    // period u-2, after its first phase there (so the copies never delay the
    // start of an MFMA phase), into ring slot u % 4, whose previous tile u-4
    // was last read in period u-3 (PV(u-4) in mfma(u-3)).
    const int grp = w >> 2;
    f32x16 sacc[2];   // S^T(t) from its MFMA phase to its softmax
    u32x4 pf[4];      // P^T(t) from its softmax to its PV
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pf[ks] = u32x4{0, 0, 0, 0};

    // The MFMA phase is 32 units (16 of PV, 16 of QK), each one LDS operand
    // fragment and one MFMA; with one wave per SIMD in this phase nothing
    // hides an LDS read's latency, so fragment u + kAhead is read while unit
    // u runs (a ring of kAhead + 1 fragments).  Lane offsets inside a tile:
    // a K fragment of k-step ks, key half kt is row kt*32 + lrow, chunk
    // (2ks + half) ^ swz(lrow & 15); a V^T fragment of k-step ks, head_dim
    // tile dt reads rows 16ks + key0 (+8), chunk 4dt + (tdb >> 3), where the
    // swizzle depends only on the row mod 16, so ks and kt enter as constants.
    constexpr int kAhead = 5;
    const int kswz = swz<D>(lrow & 15);
    const int key0 = 4 * half + (ts >> 2);
    const int vsw0 = swz<D>(key0 & 15), vsw1 = swz<D>((key0 + 8) & 15);
    const int kbase_off = lrow * kRowB;
    const int vbase0 = key0 * kRowB + (tdb & 7) * 2, vbase1 = (key0 + 8) * kRowB + (tdb & 7) * 2;
    auto read_k = [&](const char* kl, int q) PKV_INLINE -> u32x4 {  // unit 16 + q
      const int ks = q >> 1, kt = q & 1;
      return *(const u32x4*)(kl + kbase_off + kt * 32 * kRowB + (((2 * ks + half) ^ kswz) << 4));
    };
    auto read_v = [&](const char* vl, int u) PKV_INLINE -> u32x4 {  // unit u < 4 * kDTiles
      const int ks = u / kDTiles, c = 4 * (u % kDTiles) + (tdb >> 3);
      const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vl + ks * 16 * kRowB + vbase0 + ((c ^ vsw0) << 4)));
      const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vl + ks * 16 * kRowB + vbase1 + ((c ^ vsw1) << 4)));
      const u32x2 v0 = __builtin_bit_cast(u32x2, t0), v1 = __builtin_bit_cast(u32x2, t1);
      return u32x4{v0.x, v0.y, v1.x, v1.y};
    };
    auto mfma_phase = [&](int t) PKV_INLINE {
      __builtin_amdgcn_s_setprio(1);  // the MFMA stream issues first on its SIMD
      if (t >= 1) {
        // O^T += V^T P^T: the V^T operand of lane l (head_dim dt*32 + l%32,
        // keys 16*ks + 8*jj + 4*half + 0..3, jj = 0, 1) comes from two
        // transposed reads whose source lanes point at those keys' rows.
        const char* vl = I8 ? lds + kConv + (2 + ((t - 1) & 1)) * kHalfTile : lds + ((t - 1) % kStages) * kStage + kHalfTile;
        constexpr int kPvUnits = 4 * kDTiles;   // 4 k-steps of 16 keys x head_dim tiles
        u32x4 ring[kAhead + 1];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) ring[j] = read_v(vl, j);
        static_for<0, kPvUnits>([&](auto uc) PKV_INLINE {
          constexpr int u = decltype(uc)::value;
          if constexpr (u + kAhead < kPvUnits) ring[(u + kAhead) % (kAhead + 1)] = read_v(vl, u + kAhead);
          oacc[u % kDTiles] = mfma32(ring[u % (kAhead + 1)], pf[u / kDTiles], oacc[u % kDTiles]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // S^T = K Q^T for the two 32-key halves of the tile (also run on the
      // last entry, t = n, where it reads a stale slot and is never used).
      const char* kl = I8 ? lds + kConv + (t & 1) * kHalfTile : lds + (t % kStages) * kStage;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
      constexpr int kQkUnits = 2 * kKSteps;     // 2 key halves x head_dim k-steps
      u32x4 ring[kAhead + 1];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) ring[j] = read_k(kl, j);
      static_for<0, kQkUnits>([&](auto uc) PKV_INLINE {
        constexpr int q = decltype(uc)::value;
        if constexpr (q + kAhead < kQkUnits) ring[(q + kAhead) % (kAhead + 1)] = read_k(kl, q + kAhead);
        sacc[q & 1] = mfma32(ring[q % (kAhead + 1)], qf[q >> 1], sacc[q & 1]);
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_setprio(0);
    };

    auto vec_phase = [&](int t) PKV_INLINE {
      const int kv0 = t * kPfKeys;
      // Causal mask only on tiles that reach past the first row's position,
      // then the online softmax on raw dots: p = exp2(dot*|scale|*log2 e - ref).
      if (kv0 + kPfKeys - 1 > tpos0) {
        const int rel = pos_abs - kv0 - 4 * half;  // key index limit for this lane
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kt * 32 + 8 * (i >> 2) + (i & 3) > rel) sacc[kt][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kt][i]);
      tmax = pair_max(tmax) * csc;
      if (__any(tmax > m_run + kRefSlack)) {  // move the reference max (rare)
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
      const float neg_m = -m_run;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], csc, neg_m));
          sacc[kt][i] = p;
          psum += p;
        }
      l_run += psum;
      // P^T operands: k-step ks covers keys 16*ks + 8*(j/4) + 4*half + j%4,
      // j = 0..7, i.e. S^T values 8*(ks & 1) .. +7 of half ks >> 1.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, i0 = 8 * (ks & 1);
        pf[ks] = u32x4{pack_bf16(sacc[kt][i0 + 0], sacc[kt][i0 + 1]),
                       pack_bf16(sacc[kt][i0 + 2], sacc[kt][i0 + 3]),
                       pack_bf16(sacc[kt][i0 + 4], sacc[kt][i0 + 5]),
                       pack_bf16(sacc[kt][i0 + 6], sacc[kt][i0 + 7])};
      }
    };

    // Period t starts with every wave waiting for its own copies of tile t
    // and the barrier: after it tile t is complete in LDS for every wave, and
    // every wave has left period t-1.  The two groups run their sequences in
    // loops of their own, so each loop carries only the state its next phase
    // needs (P^T into group 0's MFMA phase, S^T into group 1's softmax).
    auto tile_barrier = [&](int t) PKV_INLINE {
      if constexpr (I8) {  // tile t+1's codes are in; last period's bf16 writes are done
        if (t + 2 < ntiles)
          wait_vmem<3>();
        else
          wait_vmem<0>();
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        return;
      }
      // (tile t+1's copies, kCopyLoads per wave, may stay in flight)
      if (t + 1 < ntiles)
        wait_vmem<Cf::kCopyLoads>();
      else
        wait_vmem<0>();
      // nothing moves across the barrier or a phase boundary
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (I8) {
      // As below, with the copies three tiles ahead and each wave's share of
      // the dequantisation of K(t+1) and V(t) in its VALU phase.
      if (grp == 0) {
        for (int t = 0; t <= ntiles; ++t) {
          tile_barrier(t);
          mfma_phase(t);
          if (t + 3 < ntiles) issue_tile(t + 3);
          __builtin_amdgcn_sched_barrier(0);
          if (t + 1 < ntiles) dequant(t + 1, 0);
          if (t < ntiles) {
            dequant(t, 1);
            vec_phase(t);
          }
        }
      } else {
        for (int t = 0; t <= ntiles; ++t) {
          tile_barrier(t);
          if (t >= 1) vec_phase(t - 1);
          if (t + 3 < ntiles) issue_tile(t + 3);
          if (t + 1 < ntiles) dequant(t + 1, 0);
          if (t < ntiles) dequant(t, 1);
          __builtin_amdgcn_sched_barrier(0);
          mfma_phase(t);
        }
      }
    } else if (grp == 0) {
      for (int t = 0; t <= ntiles; ++t) {
        tile_barrier(t);
        mfma_phase(t);
        if (t + 2 < ntiles) issue_tile(t + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (t < ntiles) vec_phase(t);
      }
    } else {
      for (int t = 0; t <= ntiles; ++t) {
        tile_barrier(t);
        if (t >= 1) vec_phase(t - 1);
        if (t + 2 < ntiles) issue_tile(t + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_phase(t);
      }
    }

    if (bad) tile_bad[par] = 1;
    lds_barrier();  // every wave is done with the ring; tile_bad and next_item are visible
    const bool any_bad = tile_bad[par] != 0;
    if (any_bad && tid == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);
    const float inv = any_bad ? __builtin_nanf("") : 1.f / pair_sum(l_run);
    const size_t qrow_done = qrow;
    const bool row_ok_done = row_ok;
    e = next_item[par];
    if (e < n_entries) begin_item(e);

    // Normalise and store: lane holds row lrow, head_dim elements
    // dt*32 + 8*q4 + 4*half + 0..3 (q4 = 0..3).  For each pair q4 = 2p, 2p+1
    // the two halves of the wave swap one group (v_permlane32_swap), so a
    // lane of the lower half holds dims 8*(2p) + 0..7 and a lane of the upper
    // half dims 8*(2p+1) + 0..7 of its row: one 16-byte store each.
    // (tile_bad[par] is cleared again only two items later, after barriers
    // every wave has passed.)
    uint16_t* orow = (uint16_t*)a.out + qrow_done;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const f32x16& o = oacc[dt];
        const int i0 = 8 * p2, i1 = 8 * p2 + 4;   // q4 = 2p2 and 2p2 + 1
        const uint32_t a0 = pack_bf16(o[i0 + 0] * inv, o[i0 + 1] * inv), a1 = pack_bf16(o[i0 + 2] * inv, o[i0 + 3] * inv);
        const uint32_t b0 = pack_bf16(o[i1 + 0] * inv, o[i1 + 1] * inv), b1 = pack_bf16(o[i1 + 2] * inv, o[i1 + 3] * inv);
        const auto x = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const int d = dt * 32 + 8 * (2 * p2 + half);
        if (row_ok_done) *(u32x4*)(orow + d) = u32x4{x[0], y[0], x[1], y[1]};
      }
  }
}

}  // namespace

int prefill_tile_rows(int32_t group) { return kPfRows / (group > 0 ? group : 1); }

int launch_prefill(const PrefillParams& p, int32_t head_dim, int64_t grid, hipStream_t stream) {
  if (grid <= 0 || (head_dim != 128 && !(head_dim == 64 && !p.kv_scales))) return 1;
  auto k = head_dim == 64 ? prefill_kernel<64, false, false>
           : !p.kv_scales ? prefill_kernel<128, false, false>
           : p.kv_fp8     ? prefill_kernel<128, true, true>
                          : prefill_kernel<128, true, false>;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kPfThreads), 0, stream, p, p.items, p.block_table);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
