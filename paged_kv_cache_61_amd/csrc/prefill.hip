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
//                     (the other 32 keys of the tile); exp2 with scale*log2 e
//                     folded in; rescaling skipped when no row max moved;
//   O^T += V^T P^T   (A = V^T from LDS, B = P from the S^T registers packed
//                     to bf16), so O's rows are again lane-local.
// The S^T accumulator holds keys in the order 8*(i/4) + 4*(l/32) + i%4 of the
// tile; V is written to LDS transposed ([head_dim][key]) in that same order,
// so one 16-byte LDS read gives a lane its PV operand.
// K and V tiles are gathered block by block (4 cache blocks of 16 tokens)
// with coalesced 16-byte loads into registers one tile ahead (waves 0-3 load
// K, waves 4-7 load V), then stored to a double-buffered LDS tile; row pitches are padded (K 272 B, V^T 144 B) so
// the 16-lane phases of the MFMA operand reads hit distinct banks.
// Causal masks are applied only on tiles that cross a row's position; keys
// past the chunk's last position are never loaded (zero-filled), so tail
// garbage or NaN in the cache cannot reach the output.
#include <math.h>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfRows = 256;   // MFMA rows per workgroup (8 waves x 32)
constexpr int kPfKeys = 64;    // keys per tile (4 cache blocks)
constexpr int kPfThreads = 512;
constexpr int kD = 128;        // head_dim handled by this kernel
constexpr int kKPitch = kD * 2 + 16;        // bytes per key row of the K tile
constexpr int kVPitch = kPfKeys * 2 + 16;   // bytes per head_dim row of the V^T tile
constexpr int kKTile = kPfKeys * kKPitch;   // 17408
constexpr int kVTile = kD * kVPitch;        // 18432
constexpr int kKSteps = kD / 16;            // Q.K k-steps
constexpr int kDTiles = kD / 32;            // O^T row tiles

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

// A row's reference max moves only when a tile's max exceeds it by more than
// this (log2 units); p = exp2(s - ref) stays <= 2^8 and O is rescaled rarely.
constexpr float kRefSlack = 8.f;

// LDS row of head_dim element d in the V^T tile.  The XOR spreads both the
// staging stores (rows 8 apart) and the MFMA operand reads (16 consecutive
// rows) over distinct banks with the 144-byte pitch.
PKV_DEV int vt_row(int d) { return d ^ ((d >> 4) & 7); }

// Staging registers of one thread: waves 0-3 hold K (chunk t & 15 of key
// (t >> 4) + 16 j of the tile), waves 4-7 hold V (head_dim elements
// 8*(u & 15) .. +7 of key 4*(u >> 4) + j, u = t - 256).
struct TileRegs {
  u32x4 x[4];
};

__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(PrefillParams a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * (kKTile + kVTile)];
  __shared__ int tile_bad;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index, made visibly wave-uniform so everything derived from it is scalar
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;        // which 8-wide k group of the MFMA operand
  const int lrow = lane & 31;        // MFMA row / column owned by the lane
  const int G = a.group;
  const int BQ = kPfRows / G;        // query positions per tile
  const int Hkv = a.num_kv_heads;
  const size_t row_bytes = (size_t)Hkv * kD * 2;           // bytes between token rows
  const size_t blk_bytes = kBlock * row_bytes;
  const char* kbase = (const char*)a.cache;
  const char* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  const float sl2 = a.scale_log2;
  const float csc = fabsf(sl2);

  // staging roles: waves 0-3 stage K, waves 4-7 stage V
  const bool stage_v = w >= 4;
  const int st = tid & 255;
  const int kchunk = st & 15, krow = st >> 4;     // K: chunk, key within a block
  const int vdg = st & 15, vkg = st >> 4;         // V: 8-wide head_dim group, 4-key group
  const int vwave = w - 4;                        // V: block of the tile this wave stages

  // Persistent grid over query tiles listed longest first, in serpentine
  // order (round k takes tile group k*NG + u or k*NG + NG-1-u) so the total
  // work per workgroup evens out.  Workgroup b keeps kv head b mod Hkv; with 8
  // kv heads and a grid that is a multiple of 8, workgroup b runs on XCD
  // b mod 8, so an XCD's L2 serves one head's K/V to all of its query tiles.
  const int n_entries = a.hdr[kHdrPrefillItems];
  const int wg_head = blockIdx.x % Hkv;
  const int64_t ng = gridDim.x / Hkv;            // workgroups per head
  const int64_t u = blockIdx.x / Hkv;
  const bool active = u < ng;                    // grid remainder stays idle
  for (int64_t k = 0; active; ++k) {
    const int64_t e = k * ng + ((k & 1) ? ng - 1 - u : u);
    if (e >= n_entries) break;
    const int4 item = a.items[e];
    const int g = wg_head;
    const int r = item.x, row0 = item.y, nrows = item.z;
    const int c = a.nct[r];
    const int qs = a.qsl[r];
    const int kv_end = c + row0 + nrows;               // keys 0 .. kv_end-1 are read
    const int ntiles = (kv_end + kPfKeys - 1) / kPfKeys;
    const int* bt = a.block_table + (size_t)r * a.max_blocks_per_req;

    // this lane's row
    const int rho = w * 32 + lrow;
    int pos = rho / G;
    const int head = rho - pos * G;
    const bool row_ok = rho < BQ * G && pos < nrows;
    if (!row_ok) pos = nrows - 1;                       // padding rows: any visible row
    const int pos_abs = c + row0 + pos;
    const size_t qrow = ((size_t)(qs + row0 + pos) * a.num_q_heads + g * G + head) * kD;

    // With a negative scale, q's sign is flipped (exact in bf16) and |scale|
    // used, so the row max of the raw dots is the max of the scaled scores.
    const uint32_t qsign = sl2 < 0.f ? 0x80008000u : 0u;
    u32x4 qf[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qf[ks] = row_ok ? (*(const u32x4*)((const uint16_t*)a.q + qrow + ks * 16 + 8 * half) ^ qsign)
                      : u32x4{0, 0, 0, 0};

    if (tid == 0) tile_bad = 0;
    bool bad = false;

    // Per-lane byte offsets inside a cache block (token row, kv head g, chunk).
    const uint32_t koff = krow * (uint32_t)row_bytes + g * kD * 2 + kchunk * 16;
    const uint32_t voff = 4 * (vkg & 3) * (uint32_t)row_bytes + g * kD * 2 + vdg * 16;
    // Buffer descriptor over the first `nvalid` token rows of logical block
    // b of the request: reads of rows past the chunk's last key return 0.
    auto block_rsrc = [&](const char* half_base, int b, int nvalid) {
      if (nvalid <= 0) return make_rsrc(half_base, 0);
      int phys = bt[b];
      if (phys < 0 || phys >= a.num_blocks) {
        bad = true;
        phys = 0;
      }
      return make_rsrc(half_base + (size_t)phys * blk_bytes, (uint32_t)min(nvalid, kBlock) * (uint32_t)row_bytes);
    };
    auto load_tile = [&](TileRegs& tr, int tile) {
      const int kv0 = tile * kPfKeys;
      const int b0 = kv0 / kBlock;
      if (!stage_v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase, b0 + j, kv_end - (kv0 + 16 * j));
          tr.x[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 0, 0);
        }
      } else {
        // V: wave 4+i stages block i of the tile (4 keys x 8 head_dim per lane).
        const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase, b0 + vwave, kv_end - (kv0 + 16 * vwave));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          tr.x[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + j * (uint32_t)row_bytes, 0, 0);
      }
    };

    auto store_tile = [&](const TileRegs& tr, int buf) {
      char* kl = lds + buf * (kKTile + kVTile);
      char* vl = kl + kKTile;
      if (!stage_v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4*)(kl + (16 * j + krow) * kKPitch + kchunk * 16) = tr.x[j];
      } else {
        // V^T: 4 keys of one head_dim element per 8-byte store, keys in the
        // S^T accumulator order (see the file comment).
        const int q4 = vkg & 3;
        const int col = 16 * (vkg >> 2) + 8 * (q4 & 1) + 4 * (q4 >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int word = e >> 1;
          const uint32_t x0 = tr.x[0][word], x1 = tr.x[1][word], x2 = tr.x[2][word], x3 = tr.x[3][word];
          uint32_t lo, hi;
          if (e & 1) {
            lo = __builtin_amdgcn_perm(x1, x0, 0x07060302);  // high halves of x0, x1
            hi = __builtin_amdgcn_perm(x3, x2, 0x07060302);
          } else {
            lo = __builtin_amdgcn_perm(x1, x0, 0x05040100);  // low halves of x0, x1
            hi = __builtin_amdgcn_perm(x3, x2, 0x05040100);
          }
          *(u32x2*)(vl + vt_row(8 * vdg + e) * kVPitch + col * 2) = u32x2{lo, hi};
        }
      }
    };

    f32x16 oacc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    TileRegs tr;
    load_tile(tr, 0);
    store_tile(tr, 0);
    __syncthreads();

    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      const bool more = tile + 1 < ntiles;
      if (more) load_tile(tr, tile + 1);
      const char* kl = lds + buf * (kKTile + kVTile);
      const char* vl = kl + kKTile;
      const int kv0 = tile * kPfKeys;

      // S^T = K Q^T for the two 32-key halves of the tile.
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const u32x4 kf = *(const u32x4*)(kl + (kt * 32 + lrow) * kKPitch + (ks * 16 + 8 * half) * 2);
          sacc[kt] = mfma32(kf, qf[ks], sacc[kt]);
        }

      // Causal mask only on tiles that reach past the first row's position,
      // then the online softmax on raw dots: p = exp2(dot*|scale|*log2 e - ref).
      if (kv0 + kPfKeys - 1 > c + row0) {
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
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * csc;
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

      // P^T operands: 16 keys per k-step, 8 per lane, taken from S^T values
      // 8*(ks & 1) .. +7 of half ks >> 1.
      u32x4 pf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, i0 = 8 * (ks & 1);
        pf[ks] = u32x4{pack_bf16(sacc[kt][i0 + 0], sacc[kt][i0 + 1]),
                       pack_bf16(sacc[kt][i0 + 2], sacc[kt][i0 + 3]),
                       pack_bf16(sacc[kt][i0 + 4], sacc[kt][i0 + 5]),
                       pack_bf16(sacc[kt][i0 + 6], sacc[kt][i0 + 7])};
      }
      // O^T += V^T P^T
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) {
          const u32x4 vf = *(const u32x4*)(vl + vt_row(dt * 32 + lrow) * kVPitch + (ks * 16 + 8 * half) * 2);
          oacc[dt] = mfma32(vf, pf[ks], oacc[dt]);
        }

      if (more) store_tile(tr, buf ^ 1);
      __syncthreads();
    }

    if (bad) tile_bad = 1;
    __syncthreads();
    const bool any_bad = tile_bad != 0;
    if (any_bad && tid == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);

    // Normalise and store: lane holds row lrow, head_dim elements
    // dt*32 + 8*(i/4) + 4*half + i%4.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = any_bad ? __builtin_nanf("") : 1.f / l_tot;
    if (row_ok) {
      uint16_t* orow = (uint16_t*)a.out + qrow;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = dt * 32 + 8 * q4 + 4 * half;
          const f32x16& o = oacc[dt];
          *(u32x2*)(orow + d) = u32x2{pack_bf16(o[4 * q4 + 0] * inv, o[4 * q4 + 1] * inv),
                                      pack_bf16(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv)};
        }
    }
    __syncthreads();
  }
}

}  // namespace

int prefill_tile_rows(int32_t group) { return kPfRows / (group > 0 ? group : 1); }

int launch_prefill(const PrefillParams& p, int32_t head_dim, int64_t grid, hipStream_t stream) {
  if (head_dim != kD || grid <= 0) return 1;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(kPfThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
