// Row attention over the paged cache (decode rows, split-KV partitions) and
// the split-KV merge.
//
// What is computed ("AI Infra入门干货总结：大模型是如何高效推理的", sections
// "Paged Attention" and "LLM 推理全流程" / "Attention (FlashAttention)"; the
// definition is softmax(q k^T * scale) v as in lpnh.cn/news/2669538, 2.1):
// for one query row at absolute position P of request r, every query head h
// of KV group g = h / G attends to the request's tokens 0..P, whose K/V rows
// are read from physical block block_table[r][t / 16], offset t % 16.  The G
// query heads of a group share every K/V load (GQA by index mapping).
//
// Decode is memory bound (same page, "Prefill vs Decode"): each K/V byte is
// used G times and then never again, so the kernel is built to stream the
// cache at full HBM bandwidth:
//  * a workgroup (4 waves) owns one work item = (row, kv head, partition of
//    512 tokens); wave w takes blocks w, w+4, ... of the partition and keeps
//    its own online-softmax state; the 4 states are merged through LDS;
//  * a wave reads one whole 16-token block of its kv head per step: K with
//    16-byte buffer loads in a "4 lanes per token" layout (lane = token * 4 +
//    quarter), V with one dword per lane per token in a "lanes own head_dim
//    elements" layout; both are coalesced (a K instruction covers 64
//    contiguous bytes of 16 rows, a V instruction a whole 256-byte row);
//  * the next block's loads are issued before the current block is used
//    (register double buffering); the block ids of the wave are fetched once
//    per item with one vector load and picked with readlane;
//  * q.k: per lane a partial dot over its quarter of head_dim (bf16 pairs via
//    v_dot2_f32_bf16, fp32 via FMA), finished by two quad DPP adds; the block
//    max is a row_ror DPP max plus four readlanes, so the running max m of
//    each head is wave-uniform;
//  * online softmax in the log2 domain (scale * log2 e folded into the score,
//    exp2 on the SFU); rescaling of l and o only when a block raises m;
//  * P goes through a small per-wave LDS tile to the PV layout; masked
//    positions of the last block get p = 0 and their V elements are replaced
//    by 0, so NaN or garbage in unused slots never reaches the output.
// Partitions ("Flash-Decoding", named in lpnh.cn/news/2436702 section 6)
// store (m, l, un-normalised o) per query head; the merge kernel combines
// them with the log-sum-exp rule.  The partition length is fixed, so a row's
// result does not depend on the rest of the batch.
#include <math.h>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

template <bool BF16, int D>
struct RowCfg {
  static constexpr int ES = BF16 ? 2 : 4;      // bytes per element
  static constexpr int ROWB = D * ES;          // bytes of one head's row
  static constexpr int NCH = ROWB / 16;        // 16-byte chunks per row
  static constexpr int CPL = NCH / 4;          // chunks per lane (4 lanes per token)
  static constexpr int TPI = 128 / D;          // tokens covered by one V load (2 elems/lane)
  static constexpr int VLD = kBlock / TPI;     // V loads per block per lane
};

template <bool BF16>
struct VType;
template <>
struct VType<true> {
  using T = uint32_t;
};
template <>
struct VType<false> {
  using T = u32x2;
};

template <bool BF16>
PKV_DEV float chunk_dot(const u32x4& q, const u32x4& k, float acc);

template <>
PKV_DEV float chunk_dot<true>(const u32x4& q, const u32x4& k, float acc) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}

template <>
PKV_DEV float chunk_dot<false>(const u32x4& q, const u32x4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

PKV_DEV void unpack_v(uint32_t x, float& v0, float& v1) {
  v0 = bf16_lo(x);
  v1 = bf16_hi(x);
}
PKV_DEV void unpack_v(u32x2 x, float& v0, float& v1) {
  v0 = __uint_as_float(x.x);
  v1 = __uint_as_float(x.y);
}

PKV_DEV uint32_t load_v(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
PKV_DEV u32x2 load_v(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x2) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}

PKV_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF16>
PKV_DEV void store_out(void* out, size_t idx, float x);
template <>
PKV_DEV void store_out<true>(void* out, size_t idx, float x) {
  ((uint16_t*)out)[idx] = f32_to_bf16(x);
}
template <>
PKV_DEV void store_out<false>(void* out, size_t idx, float x) {
  ((float*)out)[idx] = x;
}

template <bool BF16, int D, int GM>
__global__ __launch_bounds__(256, 2) void row_attn_kernel(RowParams a) {
  using C = RowCfg<BF16, D>;
  using VT = typename VType<BF16>::T;
  __shared__ __attribute__((aligned(16))) float p_lds[4][GM][kBlock];
  __shared__ float comb_o[4][GM][D];
  __shared__ float comb_m[4][GM];
  __shared__ float comb_l[4][GM];
  __shared__ int comb_bad[4];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int tk = lane >> 2;          // token of the block (q.k layout)
  const int cq = lane & 3;           // quarter of head_dim (q.k layout)
  const int dl = lane % (D / 2);     // element pair of head_dim (p.v layout)
  const int sub = lane / (D / 2);    // token parity when D = 64 (p.v layout)
  const int d0 = 2 * dl;

  const int n_items = a.hdr[kHdrRowItems];
  const int per_pair = a.num_kv_heads * a.head_groups;
  const int64_t total = (int64_t)n_items * per_pair;
  const uint32_t row_stride = (uint32_t)a.num_kv_heads * C::ROWB;  // bytes between token rows
  const uint32_t blk_bytes = kBlock * row_stride;
  const char* kbase = (const char*)a.cache;
  const char* vbase = kbase + (size_t)a.num_blocks * blk_bytes;

  for (int64_t it = blockIdx.x; it < total; it += gridDim.x) {
    const int4 item = a.items[it / per_pair];
    const int rem = (int)(it % per_pair);
    const int g = rem / a.head_groups;
    const int hg = rem - g * a.head_groups;
    const int h0 = g * a.group + hg * GM;
    const int nh = min(GM, a.group - hg * GM);
    const int t = item.x, r = item.y, part = item.z, slot0 = item.w;
    const size_t out_row = ((size_t)t * a.num_q_heads + h0) * D;

    if (part == kNanRow) {
      for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x)
        store_out<BF16>(a.out, out_row + idx, __builtin_nanf(""));
      continue;
    }
    const int vis = a.nct[r] + (t - a.qsl[r]) + 1;  // keys 0 .. position
    const int nblk = (vis + kBlock - 1) / kBlock;
    int jb = 0, je = nblk;
    if (part >= 0) {
      jb = part * kSplitBlocks;
      je = min(nblk, jb + kSplitBlocks);
    }

    // This lane's quarter of q for the group's heads.
    u32x4 qr[GM][C::CPL];
    const char* qrow = (const char*)a.q + out_row * C::ES;
#pragma unroll
    for (int hh = 0; hh < GM; ++hh)
#pragma unroll
      for (int k = 0; k < C::CPL; ++k)
        qr[hh][k] = hh < nh ? *(const u32x4*)(qrow + hh * C::ROWB + (cq + 4 * k) * 16)
                            : u32x4{0, 0, 0, 0};

    float m[GM], l[GM], o[GM][2];
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
      o[hh][0] = o[hh][1] = 0.f;
    }
    bool bad = false;

    const int nmine = (je - jb > w) ? (je - jb - w + 3) / 4 : 0;
    const int* bt_row = a.block_table + (size_t)r * a.max_blocks_per_req;
    const uint32_t koff = tk * row_stride + g * C::ROWB + cq * 16;
    const uint32_t voff = sub * row_stride + g * C::ROWB + d0 * C::ES;

    struct Stage {
      u32x4 k[C::CPL];
      VT v[C::VLD];
    };
    auto load = [&](Stage& s, int phys) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)phys * blk_bytes, blk_bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)phys * blk_bytes, blk_bytes);
#pragma unroll
      for (int k = 0; k < C::CPL; ++k)
        s.k[k] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + k * 64, 0, 0);
#pragma unroll
      for (int kk = 0; kk < C::VLD; ++kk) s.v[kk] = load_v(rv, voff, kk * C::TPI * row_stride, VT{});
    };
    auto compute = [&](const Stage& s, int jblk) {
      const int tok0 = jblk * kBlock;
      const bool tail = tok0 + kBlock > vis;
      float sc[GM];
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < C::CPL; ++k) acc = chunk_dot<BF16>(qr[hh][k], s.k[k], acc);
        acc += dpp_mov<kDppQuadSwap1>(acc);
        acc += dpp_mov<kDppQuadSwap2>(acc);
        sc[hh] = acc * a.scale_log2;
      }
      if (tail && tok0 + tk >= vis) {
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) sc[hh] = -INFINITY;
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        float bm = sc[hh];
        bm = fmaxf(bm, dpp_mov<kDppRowRor4>(bm));
        bm = fmaxf(bm, dpp_mov<kDppRowRor8>(bm));
        bm = fmaxf(fmaxf(readlane_f(bm, 0), readlane_f(bm, 16)),
                   fmaxf(readlane_f(bm, 32), readlane_f(bm, 48)));
        if (bm > m[hh]) {
          const float alpha = fast_exp2(m[hh] - bm);
          l[hh] *= alpha;
          o[hh][0] *= alpha;
          o[hh][1] *= alpha;
          m[hh] = bm;
        }
        const float pr = fast_exp2(sc[hh] - m[hh]);
        l[hh] += pr;
        if (cq == 0) p_lds[w][hh][(tk % C::TPI) * C::VLD + tk / C::TPI] = pr;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int kk = 0; kk < C::VLD; kk += 4) {
        float4 pv[GM];
#pragma unroll
        for (int hh = 0; hh < GM; ++hh) pv[hh] = *(const float4*)&p_lds[w][hh][sub * C::VLD + kk];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v0, v1;
          unpack_v(s.v[kk + e], v0, v1);
          if (tail && tok0 + (kk + e) * C::TPI + sub >= vis) v0 = v1 = 0.f;
#pragma unroll
          for (int hh = 0; hh < GM; ++hh) {
            const float pr = e == 0 ? pv[hh].x : e == 1 ? pv[hh].y : e == 2 ? pv[hh].z : pv[hh].w;
            o[hh][0] = fmaf(pr, v0, o[hh][0]);
            o[hh][1] = fmaf(pr, v1, o[hh][1]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    for (int kdone = 0; kdone < nmine; kdone += kWave) {
      const int nb = min(kWave, nmine - kdone);
      int btv = lane < nb ? bt_row[jb + w + 4 * (kdone + lane)] : 0;
      if (btv < 0 || btv >= a.num_blocks) {
        btv = 0;
        bad = true;
      }
      const int jfirst = jb + w + 4 * kdone;
      Stage sa, sb;
      load(sa, __builtin_amdgcn_readlane(btv, 0));
      for (int k = 0; k < nb; k += 2) {
        if (k + 1 < nb) load(sb, __builtin_amdgcn_readlane(btv, k + 1));
        compute(sa, jfirst + 4 * k);
        if (k + 1 < nb) {
          if (k + 2 < nb) load(sa, __builtin_amdgcn_readlane(btv, k + 2));
          compute(sb, jfirst + 4 * (k + 1));
        }
      }
    }

    // Wave state -> LDS.
    const bool wave_bad = __builtin_amdgcn_read_exec() != 0 && __any(bad);
#pragma unroll
    for (int hh = 0; hh < GM; ++hh) {
      l[hh] = wave_sum(l[hh]) * 0.25f;  // every token was counted by its 4 lanes
      if (C::TPI == 2) {
        o[hh][0] += __shfl_xor(o[hh][0], 32);
        o[hh][1] += __shfl_xor(o[hh][1], 32);
      }
      if (sub == 0) {
        comb_o[w][hh][d0] = o[hh][0];
        comb_o[w][hh][d0 + 1] = o[hh][1];
      }
      if (lane == 0) {
        comb_m[w][hh] = m[hh];
        comb_l[w][hh] = l[hh];
      }
    }
    if (lane == 0) comb_bad[w] = wave_bad;
    __syncthreads();
    const bool any_bad = comb_bad[0] | comb_bad[1] | comb_bad[2] | comb_bad[3];
    if (any_bad && threadIdx.x == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);
    for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
      const int hh = idx / D;
      const int d = idx - hh * D;
      float M = comb_m[0][hh];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, comb_m[ww][hh]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float f = comb_m[ww][hh] == -INFINITY ? 0.f : fast_exp2(comb_m[ww][hh] - M);
        den = fmaf(f, comb_l[ww][hh], den);
        num = fmaf(f, comb_o[ww][hh][d], num);
      }
      if (any_bad) num = __builtin_nanf("");
      if (slot0 < 0) {
        store_out<BF16>(a.out, out_row + idx, num / den);
      } else {
        const size_t s = (size_t)(slot0 + part) * a.num_q_heads + h0 + hh;
        a.part_o[s * D + d] = num;
        if (d == 0) a.part_ml[s] = make_float2(M, den);
      }
    }
    __syncthreads();
  }
}

// Merge of split-KV partitions: one wave per (row, query head).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int Hq = a.num_q_heads;
  const int64_t total = (int64_t)a.hdr[kHdrReduceItems] * Hq;
  for (int64_t it = (int64_t)blockIdx.x * 4 + w; it < total; it += (int64_t)gridDim.x * 4) {
    const int4 item = a.items[it / Hq];
    const int h = (int)(it % Hq);
    const int t = item.x, np = item.z, s0 = item.w;
    float M = -INFINITY;
    for (int p = lane; p < np; p += kWave) M = fmaxf(M, a.part_ml[(size_t)(s0 + p) * Hq + h].x);
    M = wave_max(M);
    float den = 0.f;
    float acc[D / kWave];
#pragma unroll
    for (int e = 0; e < D / kWave; ++e) acc[e] = 0.f;
    for (int p = 0; p < np; ++p) {
      const size_t s = (size_t)(s0 + p) * Hq + h;
      const float2 ml = a.part_ml[s];
      const float f = fast_exp2(ml.x - M);
      den = fmaf(f, ml.y, den);
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) acc[e] = fmaf(f, a.part_o[s * D + lane + kWave * e], acc[e]);
    }
    const size_t orow = ((size_t)t * Hq + h) * D;
#pragma unroll
    for (int e = 0; e < D / kWave; ++e) store_out<BF16>(a.out, orow + lane + kWave * e, acc[e] / den);
  }
}

template <bool BF16, int D>
int launch_rows_d(const RowParams& p, int64_t grid, hipStream_t s) {
  const int gm = p.head_groups > 1 ? kMaxGroupRegs : p.group;
  if (gm <= 1)
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, 1>), dim3(grid), dim3(256), 0, s, p);
  else if (gm <= 2)
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, 2>), dim3(grid), dim3(256), 0, s, p);
  else if (gm <= 4)
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, 4>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((row_attn_kernel<BF16, D, 8>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_rows(const RowParams& p, int32_t dtype, int32_t head_dim, int64_t grid,
                hipStream_t stream) {
  if (grid <= 0) return 0;
  const bool bf16 = dtype == PKV_BF16;
  if (head_dim == 64) return bf16 ? launch_rows_d<true, 64>(p, grid, stream)
                                  : launch_rows_d<false, 64>(p, grid, stream);
  return bf16 ? launch_rows_d<true, 128>(p, grid, stream)
              : launch_rows_d<false, 128>(p, grid, stream);
}

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
