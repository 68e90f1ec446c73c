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

// Merge of split-KV partitions: one wave per (row, query head).  With
// M = max_p m_p and f_p = exp2(m_p - M) (log2 domain), the row's output is
// sum_p f_p o_p / sum_p f_p l_p, o_p being partition p's un-normalised
// numerator.  The lanes of a wave split into PPI = 256/D groups of D/4
// lanes, each lane holding 4 consecutive head_dim elements; group j takes
// partitions j, j+PPI, ...  The loads of U*PPI partitions are issued before
// any is used (indices past the row's last partition are clamped to it and
// not added).  A row of at most 4*PPI partitions takes one such round trip,
// M included; a longer row first finds M, then merges in chunks of 4*PPI.
// Few registers keep 8 waves per SIMD resident: the merge is a chain of
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

template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void reduce_kernel(ReduceParams a) {
  constexpr int kCols = D / 4;          // float4 columns of a partial row
  constexpr int PPI = kWave / kCols;    // partitions per load instruction
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int col = lane % kCols, grp = lane / kCols;
  const int Hq = a.num_q_heads;
  const int64_t total = (int64_t)a.hdr[kHdrReduceItems] * Hq;
  for (int64_t it = (int64_t)blockIdx.x * 4 + w; it < total; it += (int64_t)gridDim.x * 4) {
    const int4 item = a.items[it / Hq];
    const int h = (int)(it % Hq);
    const int t = item.x, np = item.z, s0 = item.w;
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (np <= 4 * PPI) {
      MergeChunk<4, D> c;
      c.load(a, 0, np, s0, h, grp, col);
      const float M = wave_max(c.max_m(0, np, grp));
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
#pragma unroll
    for (int off = kCols; off < kWave; off <<= 1) {
      acc.x += __shfl_xor(acc.x, off);
      acc.y += __shfl_xor(acc.y, off);
      acc.z += __shfl_xor(acc.z, off);
      acc.w += __shfl_xor(acc.w, off);
      den += __shfl_xor(den, off);
    }
    if (grp == 0) {  // one 4-element store per lane, a whole row per group
      const size_t orow = ((size_t)t * Hq + h) * D + 4 * col;
      const float inv = 1.f / den;
      if constexpr (BF16) {
        *(uint2*)((uint16_t*)a.out + orow) =
            make_uint2((uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16),
                       (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16));
      } else {
        *(float4*)((float*)a.out + orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      }
    }
  }
}

}  // namespace

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
