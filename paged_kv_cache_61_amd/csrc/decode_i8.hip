// Row attention (decode rows, split-KV partitions, and the rows of prefill
// chunks) over an 8-bit KV cache: INT8 codes, or FP8 codes in the OCP E4M3
// format (template argument FP8).
//
// The cache holds each token's K and V rows, per kv head, as 8-bit codes with
// one float32 scale: value = code * scale, or E4M3(code) * scale (online
// quantisation of the KV cache, lpnh.cn/news/2436702 section 4.2; the rows
// are quantised as they are written, by paged_kv_write_int8 / _fp8).  Codes
// [2][num_blocks][16][Hkv][D] bytes, scales [2][num_blocks][Hkv][16] float32
// (a kv head's 16 scales of a block are contiguous).  What is computed is the same
// softmax(q k^T * scale) v over the request's tokens 0 .. position
// ("AI Infra入门干货总结", sections "Paged Attention" and "Attention
// (FlashAttention)") with k, v the dequantised rows; work items, split-KV
// partitions and the merge are those of the bf16 / fp32 row kernel.
//
// Two kernels: bf16 q runs on the matrix cores (row_attn_i8_mfma_kernel,
// below); fp32 q on the VALU kernel, per wave and 16-token block:
//  * q.k: 4 lanes per token, each over a quarter of head_dim.  A code c is
//    read as the unsigned byte u = c + 128 (one xor per 4 codes), converted
//    with v_cvt_f32_ubyte, and sum_d q_d c_d = sum_d q_d u_d - 128 sum_d q_d
//    (the q sums are taken once per item); E4M3 codes are converted exactly
//    with v_cvt_pk_f32_fp8 and need no offset.  The dot is multiplied by the
//    token's K scale; the quad adds finish it on all 4 lanes.
//  * online softmax in the log2 domain, the row max moving per block.
//  * p.v: lanes own 4 consecutive head_dim elements of D/4-lane groups; the
//    token's weight is p times its V scale (p' in LDS), and o accumulates
//    p' * u; the offset is removed at the end with the sum of the p'.
//  * the next block's codes and scales are loaded while one is used.
// Masked keys (past the row's position) get p = 0 exactly, whatever their
// codes and scales hold.
#include <math.h>

#include <algorithm>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// One work item of a wave (same lists as the bf16 / fp32 row kernel).
struct ItemI8 {
  int t, r, part, slot0;
  int g, h0, nh;
  int vis, jb, je;
};

PKV_DEV ItemI8 fetch_item_i8(const RowParams& a, int64_t it, int per_pair, int n_head, int gmax) {
  ItemI8 d;
  const int64_t e = it / per_pair;
  const int4 item = e < n_head ? load_const(a.items, e) : load_const(a.items_tail, e - n_head);
  const int rem = (int)(it % per_pair);
  d.g = rem / a.head_groups;
  const int hg = rem - d.g * a.head_groups;
  d.h0 = d.g * a.group + hg * gmax;
  d.nh = min(gmax, a.group - hg * gmax);
  d.t = item.x;
  d.r = item.y;
  d.part = item.z;
  d.slot0 = item.w;
  d.vis = d.jb = d.je = 0;
  if (d.part != kNanRow) {
    d.vis = load_const(a.nct, d.r) + (d.t - load_const(a.qsl, d.r)) + 1;
    const int nblk = (d.vis + kBlock - 1) / kBlock;
    d.je = nblk;
    if (d.part >= 0) {
      d.jb = d.part * kSplitBlocks;
      d.je = min(nblk, d.jb + kSplitBlocks);
    }
  }
  return d;
}

// u -> float for the 4 bytes of w.
PKV_DEV void ubytes(uint32_t w, float (&f)[4]) {
  f[0] = (float)(w & 0xffu);
  f[1] = (float)((w >> 8) & 0xffu);
  f[2] = (float)((w >> 16) & 0xffu);
  f[3] = (float)(w >> 24);
}

// fp32 q (bf16 q: row_attn_i8_mfma_kernel).
template <int D, int GM, bool FP8>
__global__ __launch_bounds__(256, 2) void row_attn_i8_kernel(RowParams a, const float* __restrict__ kv_scales) {
  constexpr int QPL = D / 4;          // q elements per lane (4 lanes per token)
  constexpr int KLD = QPL / 16;       // 16-byte code loads per lane per block (K)
  constexpr int VL = D / 4;           // lanes per token row in the p.v layout (4 codes each)
  constexpr int TPV = kWave / VL;     // tokens per V load
  constexpr int VLD = kBlock / TPV;   // V loads per lane per block
  __shared__ float pw_lds[4][GM][kBlock];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tk = lane >> 2, cq = lane & 3;          // q.k layout
  const int vd = lane % VL, vsub = lane / VL;       // p.v layout
  const int G = a.group;
  const int gmax = GM;
  const int per_pair = a.num_kv_heads * a.head_groups;
  const int64_t total = (int64_t)a.hdr[kHdrRowItems] * per_pair;
  const int n_head = a.hdr[kHdrRowHead];
  const uint32_t row_stride = (uint32_t)a.num_kv_heads * D;      // bytes between token rows
  const uint32_t blk_bytes = kBlock * row_stride;
  const int8_t* kbase = (const int8_t*)a.cache;
  const int8_t* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  const size_t scale_half = (size_t)a.num_blocks * kBlock * a.num_kv_heads;
  float* my_p = &pw_lds[w][0][0];
  (void)G;

  for (int64_t it = (int64_t)blockIdx.x * 4 + w; it < total; it += (int64_t)gridDim.x * 4) {
    const ItemI8 cur = fetch_item_i8(a, it, per_pair, n_head, gmax);
    const size_t out_row = ((size_t)cur.t * a.num_q_heads + cur.h0) * D;
    if (cur.part == kNanRow) {
      for (int idx = lane; idx < cur.nh * D; idx += kWave) ((float*)a.out)[out_row + idx] = __builtin_nanf("");
      continue;
    }
    const int g = cur.g, nh = cur.nh, vis = cur.vis;

    // q slice: elements cq*QPL .. +QPL-1 of each head; and its sum.
    float qr[GM][QPL];
    float qsum[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      qsum[hh] = 0.f;
      const float* src = (const float*)a.q + out_row + hh * D + cq * QPL;
#pragma unroll
      for (int j = 0; j < QPL; ++j) {
        const float x = hh < nh ? src[j] : 0.f;
        qr[hh][j] = x;
        qsum[hh] += x;
      }
    }

    float m[GM], lpart[GM], bpart[GM], o[GM][4];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      m[hh] = -INFINITY;
      lpart[hh] = bpart[hh] = 0.f;
      o[hh][0] = o[hh][1] = o[hh][2] = o[hh][3] = 0.f;
    }
    bool bad = false;

    struct Stage {
      u32x4 k[KLD];
      uint32_t v[VLD];
      float sk, sv;
    };
    const uint32_t koff = tk * row_stride + g * D + cq * QPL;
    const uint32_t voff = vsub * row_stride + g * D + 4 * vd;
    auto load = [&](Stage& s, int phys) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)phys * blk_bytes, blk_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)phys * blk_bytes, blk_bytes);
#pragma unroll
      for (int j = 0; j < KLD; ++j) s.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 16 * j, 0, 0);
#pragma unroll
      for (int j = 0; j < VLD; ++j) s.v[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, j * TPV * row_stride, kCpolNT);
      const size_t srow = ((size_t)phys * a.num_kv_heads + g) * kBlock + tk;
      s.sk = kv_scales[srow];
      s.sv = kv_scales[scale_half + srow];
    };

    auto compute = [&](const Stage& s, int jblk) {
      const int tok = jblk * kBlock + tk;
      const bool live = tok < vis;
      // q.k over this lane's quarter, offset removed, then the quad sum
      float x[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) x[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < KLD; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float f[4];
          if constexpr (FP8)
            fp8x4(s.k[j][c], f);
          else
            ubytes(s.k[j][c] ^ 0x80808080u, f);
#pragma unroll
          for (int hh = 0; hh < GM; ++hh)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[hh] = fmaf(qr[hh][16 * j + 4 * c + e], f[e], x[hh]);
        }
      }
      float sc[GM], bm[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float v = FP8 ? x[hh] : fmaf(-128.f, qsum[hh], x[hh]);
        v += dpp_mov<kDppQuadSwap1>(v);
        v += dpp_mov<kDppQuadSwap2>(v);
        sc[hh] = live ? v * (s.sk * a.scale_log2) : -INFINITY;
        // block max over the 16 tokens (lanes with the same cq)
        float b = fmaxf(sc[hh], dpp_mov<kDppRowRor4>(sc[hh]));
        b = fmaxf(b, dpp_mov<kDppRowRor8>(b));
        b = fmaxf(b, __shfl_xor(b, 16));
        bm[hh] = fmaxf(b, __shfl_xor(b, 32));
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        const float mn = fmaxf(m[hh], bm[hh]);
        const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);   // 0 on the first block
        m[hh] = mn;
        const float p = live ? __builtin_amdgcn_exp2f(sc[hh] - mn) : 0.f;
        const float pw = live ? p * s.sv : 0.f;
        lpart[hh] = lpart[hh] * alpha + (cq == 0 ? p : 0.f);
        bpart[hh] = bpart[hh] * alpha + (cq == 0 ? pw : 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[hh][e] *= alpha;
        if (cq == 0) my_p[hh * kBlock + tk] = pw;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // p.v: tokens j*TPV + vsub of the block
#pragma unroll
      for (int j = 0; j < VLD; ++j) {
        float f[4];
        if constexpr (FP8)
          fp8x4(s.v[j], f);
        else
          ubytes(s.v[j] ^ 0x80808080u, f);
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) {
          const float pw = my_p[hh * kBlock + j * TPV + vsub];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[hh][e] = fmaf(pw, f[e], o[hh][e]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // blocks jb .. je-1, ids 64 at a time, one block in flight ahead
    const int n = cur.je - cur.jb;
    const int32_t* bt = a.block_table + (size_t)cur.r * a.max_blocks_per_req;
    for (int k0 = 0; k0 < n; k0 += kWave) {
      int id = cur.jb + k0 + lane < cur.je ? bt[cur.jb + k0 + lane] : 0;
      if (id < 0 || id >= a.num_blocks) {
        id = 0;
        bad = true;
      }
      const int nb = min(kWave, n - k0);
      const int jfirst = cur.jb + k0;
      Stage sa, sb;
      load(sa, __builtin_amdgcn_readlane(id, 0));
      for (int k = 0; k < nb; k += 2) {
        if (k + 1 < nb) load(sb, __builtin_amdgcn_readlane(id, k + 1));
        compute(sa, jfirst + k);
        if (k + 1 < nb) {
          if (k + 2 < nb) load(sa, __builtin_amdgcn_readlane(id, k + 2));
          compute(sb, jfirst + k + 1);
        }
      }
    }

    // finish: sums over the wave, p.v partials over the token subsets
    const bool wave_bad = __any(bad);
    if (wave_bad && lane == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      const float l = wave_sum(lpart[hh]);
      const float bsum = wave_sum(bpart[hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int off = VL; off < kWave; off <<= 1) o[hh][e] += __shfl_xor(o[hh][e], off);
        if constexpr (!FP8) o[hh][e] = fmaf(-128.f, bsum, o[hh][e]);
      }
      if (hh < nh && vsub == 0) {
        const int d0 = 4 * vd;
        if (cur.slot0 < 0) {
          const float inv = wave_bad ? __builtin_nanf("") : 1.f / l;
          *(float4*)((float*)a.out + out_row + hh * D + d0) =
              make_float4(o[hh][0] * inv, o[hh][1] * inv, o[hh][2] * inv, o[hh][3] * inv);
        } else {
          const size_t sidx = (size_t)(cur.slot0 + cur.part) * a.num_q_heads + cur.h0 + hh;
          const float nan_or_0 = wave_bad ? __builtin_nanf("") : 0.f;
          *(float4*)(a.part_o + sidx * D + d0) =
              make_float4(o[hh][0] + nan_or_0, o[hh][1] + nan_or_0, o[hh][2] + nan_or_0, o[hh][3] + nan_or_0);
          if (vd == 0) a.part_ml[sidx] = make_float2(m[hh], l);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 q: the G query heads of a kv head share the block on the matrix cores.
//
// One wave per (query row or split-KV partition, kv head), all G <= 16 heads
// of the group in the 16 columns of 16x16 MFMA tiles (columns past G carry
// q = 0 and are not stored).  Per 16-token block:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 over head_dim/32 k-steps: A = the
//                   block's codes as exact bf16 integers (lane l: token l%16),
//                   B = q (lane l: head l%16), so lane l ends up with head l%16
//                   and tokens 4*(l/16) + 0..3 of the block;
//   scores          S * k_scale[token] * scale * log2(e); online softmax per
//                   head (the block max needs two exchanges, lanes l^16 and
//                   l^32); the reference max moves only when a block's max
//                   exceeds it by more than 2^8 (then O and l are rescaled);
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16 over head_dim/16 tiles: A = the
//                   codes of the same 4 tokens (lane l: head_dim row l%16 of
//                   each tile), B = p * v_scale[token] rounded to bf16, taken
//                   from the S^T registers as they are.
// The conversion to bf16 is exact (INT8 codes are small integers; every E4M3
// value is a bf16 value, converted two at a time by
// v_cvt_scalef32_pk_bf16_fp8 with scale 1, the V bytes of two tokens first
// paired by v_perm), the scales enter in float32; only p * v_scale is rounded
// to bf16 (relative 2^-9), as in the bf16-cache kernels.  Each lane's head_dim order inside a k-step is the same
// permutation for q and the codes (the dot product does not depend on it);
// head_dim tile dt, MFMA row r holds element (D/16)*r + dt, so a lane's output
// elements are contiguous.  Masked tokens (past the row's position, including
// unused tail slots whose codes and scales may be garbage or NaN) get p = 0
// by selection.

// Signed byte k of w as float (v_cvt_f32_i32 with a sign-extending byte select).
template <int K>
PKV_DEV float sbyte(uint32_t w) {
  return (float)(((int)w << (24 - 8 * K)) >> 24);
}
// The two E4M3 codes in the low (HI = false) or high 16 bits of w as a bf16
// pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value is a bf16
// value, so the conversion is exact).
template <bool HI>
PKV_DEV uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Two integer-valued floats (|x| < 2^8) as a bf16 pair: the top halves (exact).
PKV_DEV uint32_t ipair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302);
}

#define PKV_INLINE __attribute__((always_inline))

constexpr float kRefSlackI8 = 8.f;   // see the reference max above (log2 units)

template <int D, int NST, bool FP8>
__global__ __launch_bounds__(256, D == 128 ? 2 : 3) void row_attn_i8_mfma_kernel(RowParams a, const float* __restrict__ kv_scales) {
  constexpr int NS = D / 32;    // k-steps of S^T
  constexpr int NDT = D / 16;   // head_dim tiles of O^T = code bytes per token per lane
  constexpr int KLD = D / 64;   // 16-byte code loads per lane per block (K)
  constexpr int VW = NDT / 4;   // code dwords per token per lane (V)
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int per_pair = a.num_kv_heads * a.head_groups;
  const int64_t total = (int64_t)a.hdr[kHdrRowItems] * per_pair;
  const int n_head = a.hdr[kHdrRowHead];
  const uint32_t row_stride = (uint32_t)a.num_kv_heads * D;      // bytes between token rows
  const uint32_t blk_bytes = kBlock * row_stride;
  const int8_t* kbase = (const int8_t*)a.cache;
  const int8_t* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  const size_t scale_half = (size_t)a.num_blocks * kBlock * a.num_kv_heads;
  const float sl2 = a.scale_log2;

  // Round k of a wave takes item k*NW + gw, or k*NW + NW-1-gw in odd rounds
  // (NW waves, gw this wave's index; items are listed longest first), so a
  // wave that drew a long item in one round draws a short one in the next.
  // (Requesting the next item's descriptor and block ids while streaming the
  // current item, as the bf16 MFMA row kernel does, measured slower here.)
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  for (int64_t k = 0;; ++k) {
    const int64_t it = k * nw + ((k & 1) ? nw - 1 - gw : gw);
    if (it >= total) break;
    const ItemI8 cur = fetch_item_i8(a, it, per_pair, n_head, 16);
    const size_t out_row = ((size_t)cur.t * a.num_q_heads + cur.h0) * D;
    if (cur.part == kNanRow) {
      for (int idx = lane; idx < cur.nh * D; idx += kWave) ((uint16_t*)a.out)[out_row + idx] = 0x7fc0;
      continue;
    }
    const int g = cur.g, nh = cur.nh, vis = cur.vis;
    const bool col_ok = r16 < nh;

    // q of head r16 as the B operand: k-step s holds elements
    // 64*(s/2) + 16*q4 + 8*(s%2) + 0..7 (the codes use the same order)
    // (columns past the group read head 0's row, then zero it: no address
    // outside q is formed)
    u32x4 qb[NS];
    const uint32_t qmask = col_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4* src = (const u32x4*)((const uint16_t*)a.q + out_row + (col_ok ? r16 : 0) * D + 64 * (s >> 1) +
                                        16 * q4 + 8 * (s & 1));
      qb[s] = *src & qmask;
    }

    f32x4_t oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, lsum = 0.f;
    bool bad = false;

    struct Stage {
      u32x4 k[KLD];
      uint32_t v[4][VW];
      f32x4_t sk, sv;
    };
    // K: token r16, bytes 64j + 16*q4 .. +15 (j < KLD); V: tokens 4*q4 + i,
    // bytes NDT*r16 .. +NDT-1; the K and V scales of tokens 4*q4 .. 4*q4+3,
    // the tokens whose scores the lane holds (one 16-byte load each: a kv
    // head's 16 scales of a block are contiguous).
    const uint32_t koff = r16 * row_stride + g * D + 16 * q4;
    const uint32_t voff = 4 * q4 * row_stride + g * D + NDT * r16;
    auto load = [&](Stage& st, int phys) PKV_INLINE {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)phys * blk_bytes, blk_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)phys * blk_bytes, blk_bytes);
#pragma unroll
      for (int j = 0; j < KLD; ++j) st.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * j, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (VW == 2) {
          const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rv, voff, i * row_stride, kCpolNT);
          st.v[i][0] = x.x;
          st.v[i][1] = x.y;
        } else {
          st.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, i * row_stride, kCpolNT);
        }
      }
      const float* srow = kv_scales + ((size_t)phys * a.num_kv_heads + g) * kBlock;
      const __amdgpu_buffer_rsrc_t rsk = make_rsrc(srow, kBlock * 4);
      const __amdgpu_buffer_rsrc_t rsv = make_rsrc(srow + scale_half, kBlock * 4);
      st.sk = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsk, 16 * q4, 0, 0));
      st.sv = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsv, 16 * q4, 0, 0));
    };

    auto compute = [&](const Stage& st, int jblk) PKV_INLINE {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t c0 = st.k[s >> 1][2 * (s & 1)], c1 = st.k[s >> 1][2 * (s & 1) + 1];
        u32x4 ka;
        if constexpr (FP8)
          ka = u32x4{fp8x2_bf16<false>(c0), fp8x2_bf16<true>(c0), fp8x2_bf16<false>(c1), fp8x2_bf16<true>(c1)};
        else
          ka = u32x4{ipair(sbyte<0>(c0), sbyte<1>(c0)), ipair(sbyte<2>(c0), sbyte<3>(c0)),
                     ipair(sbyte<0>(c1), sbyte<1>(c1)), ipair(sbyte<2>(c1), sbyte<3>(c1))};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                       __builtin_bit_cast(bf16x8_t, qb[s]), sacc, 0, 0, 0);
      }
      // the lane's tokens 4*q4 + i with their own scales
      const int tok0 = jblk * kBlock + 4 * q4;
      float sc[4], vsc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vsc[i] = st.sv[i];
        sc[i] = tok0 + i < vis ? sacc[i] * (st.sk[i] * sl2) : -INFINITY;
      }
      float bmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bmax = xmax32(xmax16(bmax));
      if (__any(bmax > m_ref + kRefSlackI8)) {
        const float mn = fmaxf(m_ref, bmax);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);   // 0 on the first block
        m_ref = mn;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      }
      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[i] - m_ref);   // 0 for masked tokens
        lsum += p;
        pw[i] = tok0 + i < vis ? p * vsc[i] : 0.f;
      }
      const u32x2 pb = {__builtin_bit_cast(uint32_t, __builtin_convertvector(
                            (float __attribute__((ext_vector_type(2)))){pw[0], pw[1]}, bf16x2_t)),
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(
                            (float __attribute__((ext_vector_type(2)))){pw[2], pw[3]}, bf16x2_t))};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int wd = dt >> 2;
        u32x2 va;
        if constexpr (FP8) {
          // byte dt of tokens 0, 1 (and 2, 3) into one 16-bit half, then converted
          const uint32_t sel = (uint32_t)(dt & 3) | ((uint32_t)(4 + (dt & 3)) << 8) | 0x0c0c0000u;
          va = u32x2{fp8x2_bf16<false>(__builtin_amdgcn_perm(st.v[1][wd], st.v[0][wd], sel)),
                     fp8x2_bf16<false>(__builtin_amdgcn_perm(st.v[3][wd], st.v[2][wd], sel))};
        } else {
          float c[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = st.v[i][wd];
            c[i] = (dt & 3) == 0 ? sbyte<0>(x) : (dt & 3) == 1 ? sbyte<1>(x) : (dt & 3) == 2 ? sbyte<2>(x) : sbyte<3>(x);
          }
          va = u32x2{ipair(c[0], c[1]), ipair(c[2], c[3])};
        }
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, va),
                                                             __builtin_bit_cast(s16x4_t, pb), oacc[dt], 0, 0, 0);
      }
    };

    // blocks jb .. je-1, ids 64 at a time, NST - 1 blocks in flight ahead
    const int n = cur.je - cur.jb;
    const int32_t* bt = a.block_table + (size_t)cur.r * a.max_blocks_per_req;
    for (int k0 = 0; k0 < n; k0 += kWave) {
      int id = cur.jb + k0 + lane < cur.je ? bt[cur.jb + k0 + lane] : 0;
      if (id < 0 || id >= a.num_blocks) {
        id = 0;
        bad = true;
      }
      const int nb = min(kWave, n - k0);
      const int jfirst = cur.jb + k0;
      Stage st[NST];
#pragma unroll
      for (int j = 0; j < NST - 1; ++j)
        if (j < nb) load(st[j], __builtin_amdgcn_readlane(id, j));
      for (int k = 0; k < nb; k += NST) {
#pragma unroll
        for (int j = 0; j < NST; ++j) {
          if (k + j < nb) {
            if (k + j + NST - 1 < nb) load(st[(j + NST - 1) % NST], __builtin_amdgcn_readlane(id, k + j + NST - 1));
            compute(st[j], jfirst + k + j);
          }
        }
      }
    }

    // finish: l over the head's four lanes; lane (r16, q4) holds O elements
    // NDT*(4*q4 + i) + dt of head r16
    const bool wave_bad = __any(bad);
    if (wave_bad && lane == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);
    const float l = xsum32(xsum16(lsum));
    if (col_ok) {
      if (cur.slot0 < 0) {
        const float inv = wave_bad ? __builtin_nanf("") : 1.f / l;
        uint16_t* dst = (uint16_t*)a.out + out_row + r16 * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t pk[NDT / 2];
#pragma unroll
          for (int e = 0; e < NDT / 2; ++e)
            pk[e] = (uint32_t)f32_to_bf16(oacc[2 * e][i] * inv) | ((uint32_t)f32_to_bf16(oacc[2 * e + 1][i] * inv) << 16);
          if constexpr (NDT == 8)
            *(u32x4*)(dst + NDT * (4 * q4 + i)) = u32x4{pk[0], pk[1], pk[2], pk[3]};
          else
            *(u32x2*)(dst + NDT * (4 * q4 + i)) = u32x2{pk[0], pk[1]};
        }
      } else {
        const size_t sidx = (size_t)(cur.slot0 + cur.part) * a.num_q_heads + cur.h0 + r16;
        const float nan_or_0 = wave_bad ? __builtin_nanf("") : 0.f;
        float* dst = a.part_o + sidx * D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < NDT / 4; ++e)
            *(float4*)(dst + NDT * (4 * q4 + i) + 4 * e) =
                make_float4(oacc[4 * e][i] + nan_or_0, oacc[4 * e + 1][i] + nan_or_0, oacc[4 * e + 2][i] + nan_or_0,
                            oacc[4 * e + 3][i] + nan_or_0);
        if (q4 == 0) a.part_ml[sidx] = make_float2(m_ref, l);
      }
    }
  }
}

constexpr int kI8Stages = 3;   // register ring of blocks per wave

template <int D, bool FP8>
int launch_i8_mfma(const RowParams& p, const float* scales, int64_t bound_waves, int cus, hipStream_t s) {
  static int occ = 0;
  if (occ <= 0 && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, row_attn_i8_mfma_kernel<D, kI8Stages, FP8>, 256, 0) !=
                       hipSuccess ||
                   occ <= 0))
    occ = 2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((bound_waves + 3) / 4, (int64_t)cus * occ));
  hipLaunchKernelGGL((row_attn_i8_mfma_kernel<D, kI8Stages, FP8>), dim3((unsigned)grid), dim3(256), 0, s, p, scales);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, int GM, bool FP8>
int launch_i8_g(const RowParams& p, const float* scales, int64_t bound_waves, int cus, hipStream_t s) {
  // persistent grid: as many 4-wave workgroups as fit at once, no more than the items need
  static int occ = 0;
  if (occ <= 0 && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, row_attn_i8_kernel<D, GM, FP8>, 256, 0) !=
                       hipSuccess ||
                   occ <= 0))
    occ = 2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((bound_waves + 3) / 4, (int64_t)cus * occ));
  hipLaunchKernelGGL((row_attn_i8_kernel<D, GM, FP8>), dim3((unsigned)grid), dim3(256), 0, s, p, scales);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, bool FP8>
int launch_i8_d(const RowParams& p, const float* scales, int64_t bound_waves, int cus, hipStream_t s) {
  // fp32 q: wider groups arrive split into head groups of 2
  const int gm = p.head_groups > 1 ? 2 : p.group;
  if (gm <= 1) return launch_i8_g<D, 1, FP8>(p, scales, bound_waves, cus, s);
  if (gm <= 2) return launch_i8_g<D, 2, FP8>(p, scales, bound_waves, cus, s);
  return 1;
}

}  // namespace

int max_group_regs_i8(int32_t dtype) { return dtype == PKV_BF16 ? 16 : 2; }

template <bool FP8>
int launch_rows_fmt(const RowParams& p, const float* kv_scales, int32_t dtype, int32_t head_dim,
                    int64_t bound_waves, int cus, hipStream_t stream) {
  if (dtype == PKV_BF16)  // every group width in one wave (head_groups == 1)
    return head_dim == 64 ? launch_i8_mfma<64, FP8>(p, kv_scales, bound_waves, cus, stream)
                          : launch_i8_mfma<128, FP8>(p, kv_scales, bound_waves, cus, stream);
  if (head_dim == 64) return launch_i8_d<64, FP8>(p, kv_scales, bound_waves, cus, stream);
  return launch_i8_d<128, FP8>(p, kv_scales, bound_waves, cus, stream);
}

int launch_rows_i8(const RowParams& p, const float* kv_scales, int32_t dtype, int32_t head_dim, bool fp8,
                   int64_t bound_waves, int cus, hipStream_t stream) {
  if (bound_waves <= 0) return 0;
  return fp8 ? launch_rows_fmt<true>(p, kv_scales, dtype, head_dim, bound_waves, cus, stream)
             : launch_rows_fmt<false>(p, kv_scales, dtype, head_dim, bound_waves, cus, stream);
}

}  // namespace pkv
