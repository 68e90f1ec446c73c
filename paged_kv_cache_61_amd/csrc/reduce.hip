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

// Workgroup barrier that orders LDS accesses only (unlike __syncthreads it
// does not wait for this wave's global stores).
PKV_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// One wave merges (row t, head h) of partitions s0 .. s0 + np - 1 (np <= 4 * PPI:
// one round trip) and stores it.
template <bool BF16, int D>
PKV_DEV void merge_one(const ReduceParams& a, int t, int h, int np, int s0, int grp, int col) {
  constexpr int PPI = kWave / (D / 4);
  MergeChunk<4, D> c;
  c.load(a, 0, np, s0, h, grp, col);
  const float M = groups_max<PPI>(c.max_m(0, np, grp));
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  c.add(0, np, grp, M, acc, den);
  acc.x = groups_sum<PPI>(acc.x);
  acc.y = groups_sum<PPI>(acc.y);
  acc.z = groups_sum<PPI>(acc.z);
  acc.w = groups_sum<PPI>(acc.w);
  den = groups_sum<PPI>(den);
  if (grp == 0) store_row<BF16, D>(a, t, h, col, acc, den);
}

// Work of one launch: each wave takes groups of four query heads of the
// short rows (at most 2 * PPI partitions: two loads per head), then single
// (row, head) pairs of the other rows of at most 4 * PPI partitions; each
// workgroup then takes the (row, head) pairs of the rows with more (the
// header counts them, so a step without such rows skips that pass, and one
// with only such rows skips the per-wave pass over the rest of the list).  A
// short group issues the loads of all its heads before any is used, so it
// costs one round trip after its item is read.  Which path merges a row
// depends only on its own partition count, so a row's result does not
// depend on the rest of the batch.
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
  const int n_split = a.hdr[kHdrReduceSplit];
  const int groups = (Hq + kHeadsFast - 1) / kHeadsFast;
  const int64_t fast_units = (int64_t)n_short * groups;
  const int64_t back_units = (int64_t)(n_all - n_short) * Hq;   // rows listed from the end
  const int64_t wave_units = fast_units + (n_all - n_short > n_split ? back_units : 0);
  for (int64_t it = (int64_t)blockIdx.x * 4 + w; it < wave_units; it += (int64_t)gridDim.x * 4) {
    if (it >= fast_units) {
      const int64_t j = it - fast_units;
      const int4 item = load_const(a.items, a.cap_reduce - 1 - j / Hq);
      if (item.z <= 4 * PPI) merge_one<BF16, D>(a, item.x, (int)(j % Hq), item.z, item.w, grp, col);
      continue;   // longer rows: the workgroup pass below
    }
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
  }
  // Rows of more than 4 * PPI partitions: one workgroup per (row, query
  // head).  Wave w merges partitions [w*q, min(np, (w+1)*q)), q = ceil(np / 4),
  // against its own maximum m_w; the four partial merges then meet in LDS,
  // where wave 0 rescales each by exp2(m_w - M) and adds them in wave order,
  // so up to 16 * PPI partitions cost one round trip.
  __shared__ float4 part_acc[4][kCols];
  __shared__ float2 part_md[4];   // (m_w, denominator) of each wave's share
  const int64_t split_units = n_split > 0 ? back_units : 0;
  for (int64_t u = blockIdx.x; u < split_units; u += gridDim.x) {
    const int4 item = load_const(a.items, a.cap_reduce - 1 - u / Hq);
    const int h = (int)(u % Hq);
    const int t = item.x, np = item.z, s0 = item.w;
    if (np <= 4 * PPI) continue;   // merged by one wave in the pass above
    const int q = (np + 3) / 4;
    const int pb = min(np, w * q), nw = min(np, pb + q) - pb;
    float m = -INFINITY, den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (nw > 0) {
      if (nw <= 4 * PPI) {
        MergeChunk<4, D> c;
        c.load(a, 0, nw, s0 + pb, h, grp, col);
        m = groups_max<PPI>(c.max_m(0, nw, grp));
        c.add(0, nw, grp, m, acc, den);
      } else {
        for (int p = lane; p < nw; p += kWave) m = fmaxf(m, a.part_ml[(size_t)(s0 + pb + p) * Hq + h].x);
        m = wave_max(m);
        for (int p0 = 0; p0 < nw; p0 += 4 * PPI) {
          MergeChunk<4, D> c;
          c.load(a, p0, nw, s0 + pb, h, grp, col);
          c.add(p0, nw, grp, m, acc, den);
        }
      }
      acc.x = groups_sum<PPI>(acc.x);
      acc.y = groups_sum<PPI>(acc.y);
      acc.z = groups_sum<PPI>(acc.z);
      acc.w = groups_sum<PPI>(acc.w);
      den = groups_sum<PPI>(den);
    }
    if (grp == 0) part_acc[w][col] = acc;
    if (lane == 0) part_md[w] = make_float2(m, den);
    lds_barrier();
    if (w == 0 && grp == 0) {
      float M = part_md[0].x;
#pragma unroll
      for (int i = 1; i < 4; ++i) M = fmaxf(M, part_md[i].x);
      float dsum = 0.f;
      float4 osum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = fast_exp2(part_md[i].x - M);   // 0 for a wave with no partitions
        const float4 o = part_acc[i][col];
        dsum = fmaf(f, part_md[i].y, dsum);
        osum.x = fmaf(f, o.x, osum.x);
        osum.y = fmaf(f, o.y, osum.y);
        osum.z = fmaf(f, o.z, osum.z);
        osum.w = fmaf(f, o.w, osum.w);
      }
      store_row<BF16, D>(a, t, h, col, osum, dsum);
    }
    lds_barrier();   // the next unit rewrites part_acc / part_md
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
