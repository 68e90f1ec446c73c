// Row attention (decode rows, split-KV partitions, and the rows of prefill
// chunks) over an INT8 KV cache.
//
// The cache holds each token's K and V rows, per kv head, as int8 codes with
// one float32 scale: value = code * scale (online quantisation of the KV
// cache, lpnh.cn/news/2436702 section 4.2; the rows are quantised as they are
// written, by paged_kv_write_int8).  Codes [2][num_blocks][16][Hkv][D] int8,
// scales [2][num_blocks][16][Hkv] float32.  What is computed is the same
// softmax(q k^T * scale) v over the request's tokens 0 .. position
// ("AI Infra入门干货总结", sections "Paged Attention" and "Attention
// (FlashAttention)") with k, v the dequantised rows; work items, split-KV
// partitions and the merge are those of the bf16 / fp32 row kernel.
//
// Per wave and 16-token block:
//  * q.k: 4 lanes per token, each over a quarter of head_dim.  A code c is
//    read as the unsigned byte u = c + 128 (one xor per 4 codes), converted
//    with v_cvt_f32_ubyte, and sum_d q_d c_d = sum_d q_d u_d - 128 sum_d q_d
//    (the q sums are taken once per item).  For bf16 q the u values, exact in
//    bf16, are paired for v_dot2_f32_bf16.  The dot is multiplied by the
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
  const int4 item = e < n_head ? a.items[e] : a.items_tail[e - n_head];
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
    d.vis = a.nct[d.r] + (d.t - a.qsl[d.r]) + 1;
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

// Two small integers as float32 -> their bf16 pair (exact: < 2^8).
PKV_DEV uint32_t pair_bf16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302);
}

template <bool QBF16>
struct QSlice;
// bf16 q: the lane's D/4 elements as bf16 pairs
template <>
struct QSlice<true> {
  template <int N>
  struct Regs {
    uint32_t w[N / 2];
  };
};
template <>
struct QSlice<false> {
  template <int N>
  struct Regs {
    float w[N];
  };
};

template <bool QBF16, int D, int GM>
__global__ __launch_bounds__(256, 2) void row_attn_i8_kernel(RowParams a, const float* __restrict__ kv_scales) {
  constexpr int QPL = D / 4;          // q elements per lane (4 lanes per token)
  constexpr int KLD = QPL / 16;       // 16-byte code loads per lane per block (K)
  constexpr int VL = D / 4;           // lanes per token row in the p.v layout (4 codes each)
  constexpr int TPV = kWave / VL;     // tokens per V load
  constexpr int VLD = kBlock / TPV;   // V loads per lane per block
  using QR = typename QSlice<QBF16>::template Regs<QPL>;
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
      for (int idx = lane; idx < cur.nh * D; idx += kWave) {
        if (QBF16)
          ((uint16_t*)a.out)[out_row + idx] = 0x7fc0;
        else
          ((float*)a.out)[out_row + idx] = __builtin_nanf("");
      }
      continue;
    }
    const int g = cur.g, nh = cur.nh, vis = cur.vis;

    // q slice: elements cq*QPL .. +QPL-1 of each head; and its sum.
    QR qr[GM];
    float qsum[GM];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      qsum[hh] = 0.f;
      if constexpr (QBF16) {
        const uint32_t* src = (const uint32_t*)((const uint16_t*)a.q + out_row + hh * D + cq * QPL);
#pragma unroll
        for (int j = 0; j < QPL / 2; ++j) {
          const uint32_t x = hh < nh ? src[j] : 0u;
          qr[hh].w[j] = x;
          qsum[hh] += bf16_lo(x) + bf16_hi(x);
        }
      } else {
        const float* src = (const float*)a.q + out_row + hh * D + cq * QPL;
#pragma unroll
        for (int j = 0; j < QPL; ++j) {
          const float x = hh < nh ? src[j] : 0.f;
          qr[hh].w[j] = x;
          qsum[hh] += x;
        }
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
      for (int j = 0; j < VLD; ++j) s.v[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, j * TPV * row_stride, 0);
      const size_t srow = ((size_t)phys * kBlock + tk) * a.num_kv_heads + g;
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
          ubytes(s.k[j][c] ^ 0x80808080u, f);
#pragma unroll
          for (int hh = 0; hh < GM; ++hh) {
            if constexpr (QBF16) {
              x[hh] = dot2_bf16(qr[hh].w[8 * j + 2 * c], pair_bf16(f[0], f[1]), x[hh]);
              x[hh] = dot2_bf16(qr[hh].w[8 * j + 2 * c + 1], pair_bf16(f[2], f[3]), x[hh]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) x[hh] = fmaf(qr[hh].w[16 * j + 4 * c + e], f[e], x[hh]);
            }
          }
        }
      }
      float sc[GM], bm[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float v = fmaf(-128.f, qsum[hh], x[hh]);
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
        o[hh][e] = fmaf(-128.f, bsum, o[hh][e]);
      }
      if (hh < nh && vsub == 0) {
        const int d0 = 4 * vd;
        if (cur.slot0 < 0) {
          const float inv = wave_bad ? __builtin_nanf("") : 1.f / l;
          if constexpr (QBF16) {
            uint16_t* dst = (uint16_t*)a.out + out_row + hh * D + d0;
            *(uint2*)dst = make_uint2((uint32_t)f32_to_bf16(o[hh][0] * inv) | ((uint32_t)f32_to_bf16(o[hh][1] * inv) << 16),
                                      (uint32_t)f32_to_bf16(o[hh][2] * inv) | ((uint32_t)f32_to_bf16(o[hh][3] * inv) << 16));
          } else {
            *(float4*)((float*)a.out + out_row + hh * D + d0) =
                make_float4(o[hh][0] * inv, o[hh][1] * inv, o[hh][2] * inv, o[hh][3] * inv);
          }
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

template <bool QBF16, int D, int GM>
int launch_i8_g(const RowParams& p, const float* scales, int64_t bound_waves, int cus, hipStream_t s) {
  // persistent grid: as many 4-wave workgroups as fit at once, no more than the items need
  static int occ = 0;
  if (occ <= 0 && (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, row_attn_i8_kernel<QBF16, D, GM>, 256, 0) !=
                       hipSuccess ||
                   occ <= 0))
    occ = 2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((bound_waves + 3) / 4, (int64_t)cus * occ));
  hipLaunchKernelGGL((row_attn_i8_kernel<QBF16, D, GM>), dim3((unsigned)grid), dim3(256), 0, s, p, scales);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool QBF16, int D>
int launch_i8_d(const RowParams& p, const float* scales, int64_t bound_waves, int cus, hipStream_t s) {
  const int gm = p.head_groups > 1 ? (QBF16 ? 4 : 2) : p.group;
  if (gm <= 1) return launch_i8_g<QBF16, D, 1>(p, scales, bound_waves, cus, s);
  if (gm <= 2) return launch_i8_g<QBF16, D, 2>(p, scales, bound_waves, cus, s);
  if constexpr (QBF16) return launch_i8_g<QBF16, D, 4>(p, scales, bound_waves, cus, s);
  return 1;
}

}  // namespace

int max_group_regs_i8(int32_t dtype) { return dtype == PKV_BF16 ? 4 : 2; }

int launch_rows_i8(const RowParams& p, const float* kv_scales, int32_t dtype, int32_t head_dim,
                   int64_t bound_waves, int cus, hipStream_t stream) {
  if (bound_waves <= 0) return 0;
  const bool bf16 = dtype == PKV_BF16;
  if (head_dim == 64) return bf16 ? launch_i8_d<true, 64>(p, kv_scales, bound_waves, cus, stream)
                                  : launch_i8_d<false, 64>(p, kv_scales, bound_waves, cus, stream);
  return bf16 ? launch_i8_d<true, 128>(p, kv_scales, bound_waves, cus, stream)
              : launch_i8_d<false, 128>(p, kv_scales, bound_waves, cus, stream);
}

}  // namespace pkv
