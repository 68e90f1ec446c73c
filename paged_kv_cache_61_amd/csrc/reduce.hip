// Merge of the split-KV partitions of decode rows (the second pass of
// "Flash-Decoding", named in lpnh.cn/news/2436702 section 6): each partition
// of a row stored its running max m, denominator l and un-normalised
// numerator o per query head (decode.hip); the merge combines them with the
// log-sum-exp rule into the row's output, rounded to q's dtype.
#include <math.h>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

PKV_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge of split-KV partitions of one (row, query head).  With
// M = max_p m_p and f_p = exp2(m_p - M) (log2 domain), the row's output is
// sum_p f_p o_p / sum_p f_p l_p, o_p being partition p's un-normalised
// numerator.  The lanes of a wave split into PPI = 256/D groups of D/4
// lanes, each lane holding 4 consecutive head_dim elements; group j takes
// partitions j, j+PPI, ...  The loads of U*PPI partitions are issued before
// any is used (indices past the row's last partition are clamped to it and
// not added).  A row of at most 4*PPI partitions takes one such round trip,
// M included; a longer row first finds M, then merges in chunks of 4*PPI.
// Few registers (72) keep 7 waves per SIMD resident: the merge is a chain of
// dependent memory round trips, hidden by the other waves.
// The groups' sums are added with lane exchanges at the end.
template <int U, int D>
struct MergeChunk {
  static constexpr int PPI = kWave / (D / 4);
  float4 v[U];
  float2 ml[U];
  PKV_DEV void load(const ReduceParams& a, int p0, int np, int s0, int h, int grp, int col) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t sidx = (size_t)(s0 + min(p0 + u * PPI + grp, np - 1)) * a.num_q_heads + h;
      v[u] = ((const float4*)(a.part_o + sidx * D))[col];
      ml[u] = a.part_ml[sidx];
    }
  }
  PKV_DEV float max_m(int p0, int np, int grp) const {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (p0 + u * PPI + grp < np) m = fmaxf(m, ml[u].x);
    return m;
  }
  PKV_DEV void add(int p0, int np, int grp, float M, float4& acc, float& den) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = p0 + u * PPI + grp < np ? fast_exp2(ml[u].x - M) : 0.f;
      den = fmaf(f, ml[u].y, den);
      acc.x = fmaf(f, v[u].x, acc.x);
      acc.y = fmaf(f, v[u].y, acc.y);
      acc.z = fmaf(f, v[u].z, acc.z);
      acc.w = fmaf(f, v[u].w, acc.w);
    }
  }
};

// Store one merged row (lanes of group 0, 4 head_dim elements each).
template <bool BF16, int D>
PKV_DEV void store_row(const ReduceParams& a, int t, int h, int col, float4 acc, float den) {
  const size_t orow = ((size_t)t * a.num_q_heads + h) * D + 4 * col;
  const float inv = 1.f / den;
  if constexpr (BF16) {
    *(uint2*)((uint16_t*)a.out + orow) =
        make_uint2((uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16),
                   (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16));
  } else {
    *(float4*)((float*)a.out + orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

// Sum (or max) of the partition groups' values for every lane: groups are
// 64/PPI-lane runs, so lanes l, l ^ 16 (PPI = 4) and l ^ 32 are combined
// with v_permlane16/32 swaps (VALU).  Each step adds a pair, so the result
// is the same as that of a butterfly over __shfl_xor.
template <int PPI>
PKV_DEV float groups_sum(float x) {
  if constexpr (PPI >= 4) x = xsum16(x);
  return xsum32(x);
}
template <int PPI>
PKV_DEV float groups_max(float x) {
  if constexpr (PPI >= 4) x = xmax16(x);
  return xmax32(x);
}

// Work of one launch, in this order: groups of four query heads of each
// short row (at most 2 * PPI partitions: two loads per head), then one
// (long row, query head) at a time.  A short group issues the loads of all
// its heads before any is used, so it costs one round trip after its item
// is read; the long path is MergeChunk's.  Both add the partitions of a
// head in the same order (u ascending within a lane, then the group pairs),
// so a row's result does not depend on which path merged it.
template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void reduce_kernel(ReduceParams a) {
  constexpr int kCols = D / 4;          // float4 columns of a partial row
  constexpr int PPI = kWave / kCols;    // partitions per load instruction
  constexpr int kHeadsFast = 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int col = lane % kCols, grp = lane / kCols;
  const int Hq = a.num_q_heads;
  const int n_all = a.hdr[kHdrReduceItems], n_short = a.hdr[kHdrReduceShort];
  const int groups = (Hq + kHeadsFast - 1) / kHeadsFast;
  const int64_t fast_units = (int64_t)n_short * groups;
  const int64_t total = fast_units + (int64_t)(n_all - n_short) * Hq;
  for (int64_t it = (int64_t)blockIdx.x * 4 + w; it < total; it += (int64_t)gridDim.x * 4) {
    if (it < fast_units) {
      const int4 item = load_const(a.items, it / groups);
      const int h0 = (int)(it % groups) * kHeadsFast;
      const int t = item.x, np = item.z, s0 = item.w;
      const int nh = min(kHeadsFast, Hq - h0);
      float4 v[kHeadsFast][2];
      float2 ml[kHeadsFast][2];
#pragma unroll
      for (int hh = 0; hh < kHeadsFast; ++hh)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const size_t sidx = (size_t)(s0 + min(u * PPI + grp, np - 1)) * Hq + h0 + min(hh, nh - 1);
          v[hh][u] = ((const float4*)(a.part_o + sidx * D))[col];
          ml[hh][u] = a.part_ml[sidx];
        }
#pragma unroll
      for (int hh = 0; hh < kHeadsFast; ++hh) {
        if (hh >= nh) break;
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (u * PPI + grp < np) m = fmaxf(m, ml[hh][u].x);
        const float M = groups_max<PPI>(m);
        float den = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float f = u * PPI + grp < np ? fast_exp2(ml[hh][u].x - M) : 0.f;
          den = fmaf(f, ml[hh][u].y, den);
          acc.x = fmaf(f, v[hh][u].x, acc.x);
          acc.y = fmaf(f, v[hh][u].y, acc.y);
          acc.z = fmaf(f, v[hh][u].z, acc.z);
          acc.w = fmaf(f, v[hh][u].w, acc.w);
        }
        acc.x = groups_sum<PPI>(acc.x);
        acc.y = groups_sum<PPI>(acc.y);
        acc.z = groups_sum<PPI>(acc.z);
        acc.w = groups_sum<PPI>(acc.w);
        den = groups_sum<PPI>(den);
        if (grp == 0) store_row<BF16, D>(a, t, h0 + hh, col, acc, den);
      }
      continue;
    }
    const int64_t j = it - fast_units;
    const int4 item = load_const(a.items, a.cap_reduce - 1 - j / Hq);
    const int h = (int)(j % Hq);
    const int t = item.x, np = item.z, s0 = item.w;
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (np <= 4 * PPI) {
      MergeChunk<4, D> c;
      c.load(a, 0, np, s0, h, grp, col);
      const float M = groups_max<PPI>(c.max_m(0, np, grp));
      c.add(0, np, grp, M, acc, den);
    } else {
      float M = -INFINITY;
      for (int p = lane; p < np; p += kWave) M = fmaxf(M, a.part_ml[(size_t)(s0 + p) * Hq + h].x);
      M = wave_max(M);
      for (int p0 = 0; p0 < np; p0 += 4 * PPI) {
        MergeChunk<4, D> c;
        c.load(a, p0, np, s0, h, grp, col);
        c.add(p0, np, grp, M, acc, den);
      }
    }
    // add the groups' partial sums (den too: each group summed its own
    // partitions' weights)
    acc.x = groups_sum<PPI>(acc.x);
    acc.y = groups_sum<PPI>(acc.y);
    acc.z = groups_sum<PPI>(acc.z);
    acc.w = groups_sum<PPI>(acc.w);
    den = groups_sum<PPI>(den);
    if (grp == 0) store_row<BF16, D>(a, t, h, col, acc, den);  // one 4-element store per lane
  }
}

}  // namespace

int reduce_short_parts(int32_t head_dim) { return 2 * (kWave / (head_dim / 4)); }

int launch_reduce(const ReduceParams& p, int32_t dtype, int32_t head_dim, int64_t grid,
                  hipStream_t stream) {
  if (grid <= 0) return 0;
  const bool bf16 = dtype == PKV_BF16;
  if (head_dim == 64) {
    if (bf16)
      hipLaunchKernelGGL((reduce_kernel<true, 64>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((reduce_kernel<false, 64>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (bf16)
      hipLaunchKernelGGL((reduce_kernel<true, 128>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((reduce_kernel<false, 128>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
