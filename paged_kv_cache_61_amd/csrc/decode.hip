// Row attention over the paged cache (decode rows, split-KV partitions).
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
//  * a work item is (row, kv head, partition of 1024 tokens); every wave is an
//    independent persistent worker that takes items in a fixed interleaved
//    order and streams all blocks of its item itself (the 4 waves of a
//    workgroup share nothing but the CU; each has its own small LDS tile);
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
// store (m, l, un-normalised o) per query head; the merge kernel (reduce.hip) combines
// them with the log-sum-exp rule.  The partition length is fixed, so a row's
// result does not depend on the rest of the batch.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

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

PKV_DEV void unpack_v(u32x2 x, float& v0, float& v1) {
  v0 = __uint_as_float(x.x);
  v1 = __uint_as_float(x.y);
}

PKV_DEV uint32_t load_v(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCpolNT);
}
PKV_DEV u32x2 load_v(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x2) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCpolNT);
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

// out[idx], out[idx + 1] = x0, x1 in one store (idx even).
template <bool BF16>
PKV_DEV void store_out2(void* out, size_t idx, float x0, float x1) {
  if constexpr (BF16)
    *(uint32_t*)((uint16_t*)out + idx) = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
  else
    *(float2*)((float*)out + idx) = make_float2(x0, x1);
}

// Lanes that share one token's q.k: 4, each owning a quarter of head_dim.  A
// wave holds 1, 2 or 4 query heads of a group (wider groups are split into
// several waves of 4 heads by the host).
template <int GM>
struct Lanes {
  static_assert(GM == 1 || GM == 2 || GM == 4, "a wave holds 1, 2 or 4 heads");
  static constexpr int kPerToken = 4;
  static constexpr int kTokensPerPass = kWave / kPerToken;   // 16
  static constexpr int kPasses = kBlock / kTokensPerPass;      // 1
  static constexpr int kHeadsPerLane = GM > kPerToken ? GM / kPerToken : 1;
  // head held by lane quarter/eighth c in slot k after the reduce-scatter
  PKV_DEV static int head(int c, int k) {
    return GM >= kPerToken ? c + kPerToken * k : (GM == 2 ? (c & 1) : 0);
  }
  // one lane per distinct head writes shared per-head values
  PKV_DEV static bool writer(int c) { return c < (GM < kPerToken ? GM : kPerToken); }
};

// Sum the partial dots x[0..GM) over the lanes of a token so that lane c ends
// with the full dots of its Lanes<GM>::head(c, k) heads in y[].  Each DPP step
// halves the heads a lane keeps: the lane keeps one half and adds what its
// partner sends of that half.
template <int GM>
PKV_DEV void reduce_scatter(const float (&x)[GM], float (&y)[Lanes<GM>::kHeadsPerLane], int c) {
  if constexpr (GM == 1) {
    const float v = x[0] + dpp_mov<kDppQuadSwap1>(x[0]);
    y[0] = v + dpp_mov<kDppQuadSwap2>(v);
  } else if constexpr (GM == 2) {
    const bool b = c & 1;
    const float v = (b ? x[1] : x[0]) + dpp_mov<kDppQuadSwap1>(b ? x[0] : x[1]);
    y[0] = v + dpp_mov<kDppQuadSwap2>(v);
  } else {  // GM == 4
    const bool b0 = c & 1, b1 = (c >> 1) & 1;
    float x1[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      x1[j] = (b0 ? x[2 * j + 1] : x[2 * j]) + dpp_mov<kDppQuadSwap1>(b0 ? x[2 * j] : x[2 * j + 1]);
    y[0] = (b1 ? x1[1] : x1[0]) + dpp_mov<kDppQuadSwap2>(b1 ? x1[0] : x1[1]);
  }
}

// Max / sum over the tokens of one pass for lanes sharing c (lane = token *
// LPT + c): rotate within 16-lane rows, then exchange across rows.
template <int LPT>
PKV_DEV float pass_max(float v) {
  if constexpr (LPT == 4) v = fmaxf(v, dpp_mov<kDppRowRor4>(v));
  v = fmaxf(v, dpp_mov<kDppRowRor8>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
template <int LPT>
PKV_DEV float pass_sum(float v) {
  if constexpr (LPT == 4) v += dpp_mov<kDppRowRor4>(v);
  v += dpp_mov<kDppRowRor8>(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// A head's reference max moves only when a score exceeds it by more than
// this (log2 units), so p = exp2(s - ref) <= 2^8.  Numerator and denominator
// share the reference, so the softmax stays exact.
constexpr float kRefSlack = 8.f;

// What a wave needs to know about one work item.
struct RowItem {
  int t, r, part, slot0;   // query row, request, partition (or kWholeRow / kNanRow), first slot
  int g, h0, nh;           // kv head, first query head, heads handled
  int vis, jb, je;         // visible keys, block range [jb, je)
};

template <int GM>
PKV_DEV RowItem fetch_item(const RowParams& a, int64_t it, int per_pair, int n_head) {
  RowItem d;
  const int64_t e = it / per_pair;
  const int4 item = e < n_head ? load_const(a.items, e) : load_const(a.items_tail, e - n_head);
  const int rem = (int)(it % per_pair);
  d.g = rem / a.head_groups;
  const int hg = rem - d.g * a.head_groups;
  d.h0 = d.g * a.group + hg * GM;
  d.nh = min(GM, a.group - hg * GM);
  d.t = item.x;
  d.r = item.y;
  d.part = item.z;
  d.slot0 = item.w;
  d.vis = d.jb = d.je = 0;
  if (d.part != kNanRow) {
    d.vis = load_const(a.nct, d.r) + (d.t - load_const(a.qsl, d.r)) + 1;  // keys 0 .. position
    const int nblk = (d.vis + kBlock - 1) / kBlock;
    d.je = nblk;
    if (d.part >= 0) {
      d.jb = d.part * kSplitBlocks;
      d.je = min(nblk, d.jb + kSplitBlocks);
    }
  }
  return d;
}

// Lane j gets the physical id of block jb + k0 + j of the item (j < 64).
PKV_DEV int fetch_ids(const RowParams& a, const RowItem& d, int k0, int lane) {
  const int j = d.jb + k0 + lane;
  return j < d.je ? a.block_table[(size_t)d.r * a.max_blocks_per_req + j] : 0;
}

// Each wave is an independent persistent worker: in round k it takes item
// k*NW + gw or, in odd rounds, k*NW + NW-1-gw (gw = global wave index, NW =
// waves in the grid; items are listed longest first), and while it streams
// one item's blocks it already holds the next item's descriptor and block
// ids, so switching items costs one memory round trip.  Consecutive items
// (the heads of one partition) go to adjacent waves of one workgroup, so a CU
// reads adjacent head rows together.
// (A shared atomic work counter was measured slower: claims serialise on one
// address.)
template <bool BF16, int D, int GM>
__global__ __launch_bounds__(256, !BF16 && D == 128 ? 1 : 2) void row_attn_kernel(RowParams a) {
  using C = RowCfg<BF16, D>;
  using VT = typename VType<BF16>::T;
  using LN = Lanes<GM>;
  constexpr int LPT = LN::kPerToken;
  constexpr int TPP = LN::kTokensPerPass;
  constexpr int NPASS = LN::kPasses;
  constexpr int HPL = LN::kHeadsPerLane;
  constexpr int CPL = C::NCH / LPT;      // 16-byte chunks of a row per lane
  constexpr int PSZ = BF16 ? 2 : 4;      // bytes of one p value in LDS
  __shared__ __attribute__((aligned(16))) char p_lds[4][GM * kBlock * PSZ];
  __shared__ float alpha_lds[4][GM];
  __shared__ float2 ml_lds[4][GM];

  const int lane = threadIdx.x & (kWave - 1);
  // wave index, made visibly wave-uniform so everything derived from it is scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tk = lane / LPT;         // token of the pass (q.k layout)
  const int cq = lane % LPT;         // slice of head_dim (q.k layout)
  const int dl = lane % (D / 2);     // element pair of head_dim (p.v layout)
  const int sub = lane / (D / 2);    // token parity when D = 64 (p.v layout)
  const int d0 = 2 * dl;

  const int per_pair = a.num_kv_heads * a.head_groups;
  const int64_t total = (int64_t)a.hdr[kHdrRowItems] * per_pair;
  const int n_head = a.hdr[kHdrRowHead];
  const uint32_t row_stride = (uint32_t)a.num_kv_heads * C::ROWB;  // bytes between token rows
  const uint32_t blk_bytes = kBlock * row_stride;
  const char* kbase = (const char*)a.cache;
  const char* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  char* my_p = p_lds[w];

  // Serpentine order over the longest-first list: round k takes item
  // k*NW + gw (k even) or k*NW + NW-1-gw (k odd), which balances the total
  // work per wave like longest-processing-time-first.
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  auto item_of = [&](int64_t k) { return k * nw + ((k & 1) ? nw - 1 - gw : gw); };
  int64_t round = 0;
  const int64_t it = item_of(0);
  if (it >= total) return;
  int64_t nx = item_of(1);
  RowItem cur = fetch_item<GM>(a, it, per_pair, n_head);
  int btv = fetch_ids(a, cur, 0, lane);

  while (true) {
    const bool has_next = nx < total;
    const int64_t nx2 = item_of(round + 2);
    RowItem nxt = cur;
    int btv_next = 0;
    if (has_next) {  // prefetch: consumed only after this item
      nxt = fetch_item<GM>(a, nx, per_pair, n_head);
      btv_next = fetch_ids(a, nxt, 0, lane);
    }
    const size_t out_row = ((size_t)cur.t * a.num_q_heads + cur.h0) * D;

    if (cur.part == kNanRow) {
      for (int idx = lane; idx < cur.nh * D; idx += kWave)
        store_out<BF16>(a.out, out_row + idx, __builtin_nanf(""));
    } else {
      const int g = cur.g, nh = cur.nh, vis = cur.vis;
      // This lane's slice of q for the group's heads: chunks cq + LPT * k.
      u32x4 qr[GM][CPL];
      const char* qrow = (const char*)a.q + out_row * C::ES;
#pragma unroll
      for (int hh = 0; hh < GM; ++hh)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
          qr[hh][k] = hh < nh ? *(const u32x4*)(qrow + hh * C::ROWB + (cq + LPT * k) * 16)
                              : u32x4{0, 0, 0, 0};

      float mref[HPL], lsum[HPL], o[GM][2];
#pragma unroll
      for (int k = 0; k < HPL; ++k) {
        mref[k] = -INFINITY;
        lsum[k] = 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) o[hh][0] = o[hh][1] = 0.f;
      bool bad = false;

      const uint32_t koff = tk * row_stride + g * C::ROWB + cq * 16;
      const uint32_t voff = sub * row_stride + g * C::ROWB + d0 * C::ES;

      struct Stage {
        u32x4 k[NPASS][CPL];
        VT v[C::VLD];
      };
      auto load = [&](Stage& s, int phys) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)phys * blk_bytes, blk_bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)phys * blk_bytes, blk_bytes);
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
          for (int k = 0; k < CPL; ++k)
            s.k[ps][k] = __builtin_amdgcn_raw_buffer_load_b128(
                rk, koff + ps * TPP * row_stride + k * LPT * 16, 0, 0);
#pragma unroll
        for (int kk = 0; kk < C::VLD; ++kk) s.v[kk] = load_v(rv, voff, kk * C::TPI * row_stride, VT{});
      };

      auto compute = [&](auto mask_tag, const Stage& s, int jblk) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int tok0 = jblk * kBlock;
        float sc[NPASS][HPL];
        bool raise = false;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          // q.k partial dots over this lane's slice, then reduce-scatter.
          float x[GM];
#pragma unroll
          for (int hh = 0; hh < GM; ++hh) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) acc = chunk_dot<BF16>(qr[hh][k], s.k[ps][k], acc);
            x[hh] = acc;
          }
          reduce_scatter<GM>(x, sc[ps], cq);
          const bool live = !MASK || tok0 + ps * TPP + tk < vis;
#pragma unroll
          for (int k = 0; k < HPL; ++k) {
            sc[ps][k] = live ? sc[ps][k] * a.scale_log2 : -INFINITY;
            raise |= sc[ps][k] > mref[k] + kRefSlack;
          }
        }
        const bool rescale = __any(raise);
        if (rescale) {  // rare: move the reference max
#pragma unroll
          for (int k = 0; k < HPL; ++k) {
            float bm = sc[0][k];
#pragma unroll
            for (int ps = 1; ps < NPASS; ++ps) bm = fmaxf(bm, sc[ps][k]);
            const float mnew = fmaxf(mref[k], pass_max<LPT>(bm));
            const float alpha = __builtin_amdgcn_exp2f(mref[k] - mnew);
            lsum[k] *= alpha;
            mref[k] = mnew;
            if (tk == 0 && LN::writer(cq)) alpha_lds[w][LN::head(cq, k)] = alpha;
          }
        }
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
          for (int k = 0; k < HPL; ++k) {
            const float p = __builtin_amdgcn_exp2f(sc[ps][k] - mref[k]);
            const int hh = LN::head(cq, k);
            const int tb = ps * TPP + tk;  // token of the block
            const int pidx = (hh * C::TPI + tb % C::TPI) * C::VLD + tb / C::TPI;
            if constexpr (BF16) {
              const uint16_t pb = f32_to_bf16(p);
              lsum[k] += __uint_as_float((uint32_t)pb << 16);
              if (LN::writer(cq)) ((uint16_t*)my_p)[pidx] = pb;
            } else {
              lsum[k] += p;
              if (LN::writer(cq)) ((float*)my_p)[pidx] = p;
            }
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (rescale) {
#pragma unroll
          for (int hh = 0; hh < GM; ++hh) {
            const float al = alpha_lds[w][hh];
            o[hh][0] *= al;
            o[hh][1] *= al;
          }
        }
        // p.v: lanes own head_dim pairs; tokens kk*TPI + sub.
        if constexpr (BF16) {
#pragma unroll
          for (int j = 0; j < C::VLD / 2; j += 2) {
            u32x2 pp[GM];
#pragma unroll
            for (int hh = 0; hh < GM; ++hh)
              pp[hh] = *(const u32x2*)(my_p + ((hh * C::TPI + sub) * C::VLD + 2 * j) * 2);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              uint32_t x0 = s.v[2 * (j + e)], x1 = s.v[2 * (j + e) + 1];
              if constexpr (MASK) {
                if (tok0 + (2 * (j + e)) * C::TPI + sub >= vis) x0 = 0;
                if (tok0 + (2 * (j + e) + 1) * C::TPI + sub >= vis) x1 = 0;
              }
              const uint32_t vd0 = __builtin_amdgcn_perm(x1, x0, 0x05040100);
              const uint32_t vd1 = __builtin_amdgcn_perm(x1, x0, 0x07060302);
#pragma unroll
              for (int hh = 0; hh < GM; ++hh) {
                const uint32_t p2 = pp[hh][e];
                o[hh][0] = dot2_bf16(p2, vd0, o[hh][0]);
                o[hh][1] = dot2_bf16(p2, vd1, o[hh][1]);
              }
            }
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < C::VLD; kk += 4) {
            float4 pv[GM];
#pragma unroll
            for (int hh = 0; hh < GM; ++hh)
              pv[hh] = *(const float4*)(my_p + ((hh * C::TPI + sub) * C::VLD + kk) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v0, v1;
              unpack_v(s.v[kk + e], v0, v1);
              if constexpr (MASK) {
                if (tok0 + (kk + e) * C::TPI + sub >= vis) v0 = v1 = 0.f;
              }
#pragma unroll
              for (int hh = 0; hh < GM; ++hh) {
                const float pr = e == 0 ? pv[hh].x : e == 1 ? pv[hh].y : e == 2 ? pv[hh].z : pv[hh].w;
                o[hh][0] = fmaf(pr, v0, o[hh][0]);
                o[hh][1] = fmaf(pr, v1, o[hh][1]);
              }
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
      auto step = [&](const Stage& s, int jblk) {
        if (jblk * kBlock + kBlock > vis)
          compute(std::true_type{}, s, jblk);
        else
          compute(std::false_type{}, s, jblk);
      };

      // Blocks jb .. je-1, 64 ids at a time (split items have at most 32).
      const int n = cur.je - cur.jb;
      for (int k0 = 0; k0 < n; k0 += kWave) {
        if (k0 > 0) btv = fetch_ids(a, cur, k0, lane);
        if (btv < 0 || btv >= a.num_blocks) {
          btv = 0;
          bad = true;
        }
        const int nb = min(kWave, n - k0);
        const int jfirst = cur.jb + k0;
        Stage sa, sb;
        load(sa, __builtin_amdgcn_readlane(btv, 0));
        if (nb > 1) load(sb, __builtin_amdgcn_readlane(btv, 1));
        for (int k = 0; k < nb; k += 2) {
          step(sa, jfirst + k);
          if (k + 2 < nb) load(sa, __builtin_amdgcn_readlane(btv, k + 2));
          if (k + 1 < nb) {
            step(sb, jfirst + k + 1);
            if (k + 3 < nb) load(sb, __builtin_amdgcn_readlane(btv, k + 3));
          }
        }
      }

      // Finish: per-head (m, l) through LDS, then out or the partial.
      const bool wave_bad = __any(bad);
#pragma unroll
      for (int k = 0; k < HPL; ++k) {
        const float lt = pass_sum<LPT>(lsum[k]);
        if (tk == 0 && LN::writer(cq)) ml_lds[w][LN::head(cq, k)] = make_float2(mref[k], lt);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (wave_bad && lane == 0) atomicOr(a.err, PKV_DEVERR_BLOCK_ID);
#pragma unroll
      for (int hh = 0; hh < GM; ++hh) {
        if (C::TPI == 2) {
          o[hh][0] += __shfl_xor(o[hh][0], 32);
          o[hh][1] += __shfl_xor(o[hh][1], 32);
        }
        if (hh < nh && sub == 0) {
          const float2 ml = ml_lds[w][hh];
          if (cur.slot0 < 0) {
            const float inv = wave_bad ? __builtin_nanf("") : 1.f / ml.y;
            store_out2<BF16>(a.out, out_row + hh * D + d0, o[hh][0] * inv, o[hh][1] * inv);
          } else {
            const size_t sidx = (size_t)(cur.slot0 + cur.part) * a.num_q_heads + cur.h0 + hh;
            const float nan_or_0 = wave_bad ? __builtin_nanf("") : 0.f;
            *(float2*)(a.part_o + sidx * D + d0) = make_float2(o[hh][0] + nan_or_0, o[hh][1] + nan_or_0);
            if (dl == 0) a.part_ml[sidx] = ml;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (!has_next) break;
    ++round;
    nx = nx2;
    cur = nxt;
    btv = btv_next;
  }
}

// bf16 q and cache on the matrix cores: one wave per (row or partition, kv
// head) with all G <= 16 query heads of the group in the 16 columns of 16x16
// MFMA tiles (columns past G carry q = 0 and are not stored), so a block is
// read once and its dot products cost a few MFMAs whatever G is.  Per block:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 over head_dim/32 k-steps, the
//                   A operand straight from the loaded rows (lane l: token
//                   l%16, elements 32s + 8*(l/16) .. +7 of k-step s), B = q of
//                   head l%16 (same elements), so lane l ends up with head
//                   l%16 and tokens 4*(l/16) + 0..3;
//   online softmax  per head in the log2 domain, the block max over two
//                   lane exchanges (l^16, l^32), the reference max moving only
//                   when a block's max exceeds it by more than 2^8; p rounded
//                   to bf16 for the product and added to l as rounded;
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16 over head_dim/16 tiles: A = V of
//                   the same 4 tokens (lane l: element (D/16)*(l%16) + dt of
//                   tile dt, two half-word permutes per tile), B = P^T from the
//                   S^T registers as they are.
// Masked tokens (past the row's position) get p = 0 by selection and their V
// rows are zeroed before the product, so NaN in unused slots never reaches
// the output.  Items are visited in the serpentine order of row_attn_kernel,
// with the next item's descriptor and block ids fetched while one streams.
template <int D>
__global__ __launch_bounds__(256, 2) void row_attn_mfma_kernel(RowParams a) {
  constexpr int NS = D / 32;    // k-steps of S^T = 16-byte K loads per lane per block
  constexpr int NDT = D / 16;   // head_dim tiles of O^T = V elements per token per lane
  constexpr int ROWB = D * 2;
  constexpr int NST = 2;        // register ring of blocks
  typedef typename std::conditional<NDT == 8, u32x4, u32x2>::type VRow;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int per_pair = a.num_kv_heads * a.head_groups;
  const int64_t total = (int64_t)a.hdr[kHdrRowItems] * per_pair;
  const int n_head = a.hdr[kHdrRowHead];
  const uint32_t row_stride = (uint32_t)a.num_kv_heads * ROWB;
  const uint32_t blk_bytes = kBlock * row_stride;
  const char* kbase = (const char*)a.cache;
  const char* vbase = kbase + (size_t)a.num_blocks * blk_bytes;
  const float sl2 = a.scale_log2;

  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  auto item_of = [&](int64_t k) { return k * nw + ((k & 1) ? nw - 1 - gw : gw); };
  int64_t round = 0;
  const int64_t it = item_of(0);
  if (it >= total) return;
  int64_t nx = item_of(1);
  // Block ids outside the pool are replaced by block 0 (and reported).  Each
  // id vector is checked right where it is fetched or where every earlier
  // load has landed anyway, so no later use of it waits on the stream.
  auto check_ids = [&](int& ids) __attribute__((always_inline)) -> bool {
    const bool out = ids < 0 || ids >= a.num_blocks;
    if (out) ids = 0;
    return out;
  };
  RowItem cur = fetch_item<16>(a, it, per_pair, n_head);
  int btv = fetch_ids(a, cur, 0, lane);
  bool btv_bad = check_ids(btv);

  struct Stage {
    u32x4 k[NS];
    VRow v[4];
  };
  static_assert(NST == 2, "one block computed while the next one loads");
  // kv head g's part of a block: K token r16, elements 16*q4 + 64*s (k-step
  // s); V tokens 4*q4 + i, elements 2*NDT*r16 .. (byte offsets)
  auto koff_of = [&](int g) -> uint32_t { return r16 * row_stride + g * ROWB + 16 * q4; };
  auto voff_of = [&](int g) -> uint32_t { return 4 * q4 * row_stride + g * ROWB + 2 * NDT * r16; };
  auto load = [&](Stage& st, int phys, uint32_t koff, uint32_t voff) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (size_t)phys * blk_bytes, blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (size_t)phys * blk_bytes, blk_bytes);
#pragma unroll
    for (int s = 0; s < NS; ++s) st.k[s] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * s, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (NDT == 8)
        st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, i * row_stride, kCpolNT);
      else
        st.v[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, voff, i * row_stride, kCpolNT);
    }
  };
  // q of head r16 of an item as the B operand (k-step s: elements 32s + 8*q4
  // .. +7, the order of the K rows).  Columns past the group read head 0's
  // row: a column's scores, softmax state and output stay in that column of
  // both products and are never stored, so the rows need no masking (and
  // nothing waits for q before the block stream starts).
  auto load_q = [&](u32x4 (&qb)[NS], const RowItem& d) __attribute__((always_inline)) {
    const size_t row = ((size_t)d.t * a.num_q_heads + d.h0 + (r16 < d.nh ? r16 : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = *(const u32x4*)((const uint16_t*)a.q + row + 32 * s + 8 * q4);
  };

  while (true) {
    const bool has_next = nx < total;
    const int64_t nx2 = item_of(round + 2);
    RowItem nxt = cur;
    int btv_next = 0;
    bool btv_next_bad = false;
    // The next item's descriptor and block ids (dependent loads: item ->
    // request metadata -> block table) are consumed only after this item.
    // They are requested once this item's first block is in flight, so their
    // round trips overlap that block's instead of preceding it.
    auto fetch_next = [&]() __attribute__((always_inline)) {
      if (has_next) {
        nxt = fetch_item<16>(a, nx, per_pair, n_head);
        btv_next = fetch_ids(a, nxt, 0, lane);
      }
    };
    const size_t out_row = ((size_t)cur.t * a.num_q_heads + cur.h0) * D;
    if (cur.part == kNanRow) {
      fetch_next();
      btv_next_bad = check_ids(btv_next);
      for (int idx = lane; idx < cur.nh * D; idx += kWave) ((uint16_t*)a.out)[out_row + idx] = 0x7fc0;
    } else {
      const int g = cur.g, nh = cur.nh, vis = cur.vis;
      const bool col_ok = r16 < nh;
      u32x4 qb[NS];
      load_q(qb, cur);

      f32x4_t oacc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float m_ref = -INFINITY, lsum = 0.f;
      bool bad = btv_bad;
      const uint32_t koff = koff_of(g), voff = voff_of(g);

      auto compute = [&](const Stage& st, int jblk) __attribute__((always_inline)) {
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, st.k[s]),
                                                         __builtin_bit_cast(bf16x8_t, qb[s]), sacc, 0, 0, 0);
        const int tok0 = jblk * kBlock + 4 * q4;
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = tok0 + i < vis ? sacc[i] * sl2 : -INFINITY;
        float bmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        bmax = xmax32(xmax16(bmax));
        if (__any(bmax > m_ref + kRefSlack)) {
          const float mn = fmaxf(m_ref, bmax);
          const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);   // 0 on the first block
          m_ref = mn;
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        }
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = f32_to_bf16(__builtin_amdgcn_exp2f(sc[i] - m_ref));   // 0 for masked tokens
          lsum += __uint_as_float(pb[i] << 16);
        }
        const u32x2 pt = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
        uint32_t vw[4][NDT / 2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < NDT / 2; ++e) vw[i][e] = st.v[i][e];
        if (jblk * kBlock + kBlock > vis) {   // the row's last block: zero V past the position
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tok0 + i >= vis)
#pragma unroll
              for (int e = 0; e < NDT / 2; ++e) vw[i][e] = 0u;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
          const u32x2 va = {__builtin_amdgcn_perm(vw[1][dt >> 1], vw[0][dt >> 1], sel),
                            __builtin_amdgcn_perm(vw[3][dt >> 1], vw[2][dt >> 1], sel)};
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, va),
                                                               __builtin_bit_cast(s16x4_t, pt), oacc[dt], 0, 0, 0);
        }
      };

      // Blocks jb .. je-1, 64 ids at a time, the next block always in flight
      // (items of more than 64 blocks, whole rows without split-KV, fetch
      // each further 64 ids when they reach them).
      const int n = cur.je - cur.jb;
      Stage st[NST];
      int btv_c = btv;
      for (int k0 = 0; k0 < n; k0 += kWave) {
        if (k0 > 0) {
          btv_c = fetch_ids(a, cur, k0, lane);
          bad |= check_ids(btv_c);
        }
        const int nb = min(kWave, n - k0);
        const int jfirst = cur.jb + k0;
        load(st[0], __builtin_amdgcn_readlane(btv_c, 0), koff, voff);
        if (k0 == 0) fetch_next();
        for (int k = 0; k < nb; k += 2) {
          if (k + 1 < nb) load(st[1], __builtin_amdgcn_readlane(btv_c, k + 1), koff, voff);
          compute(st[0], jfirst + k);
          if (k + 1 < nb) {
            if (k + 2 < nb) load(st[0], __builtin_amdgcn_readlane(btv_c, k + 2), koff, voff);
            compute(st[1], jfirst + k + 1);
          }
        }
      }
      if (n <= 0) fetch_next();
      // (every load of this item has landed: checking the next ids here
      // waits for nothing, and the next item's first loads wait for nothing)
      btv_next_bad = check_ids(btv_next);

      // Finish: l over the head's four lanes; lane (r16, q4) holds O
      // elements NDT*(4*q4 + i) + dt of head r16.
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
                  make_float4(oacc[4 * e][i] + nan_or_0, oacc[4 * e + 1][i] + nan_or_0,
                              oacc[4 * e + 2][i] + nan_or_0, oacc[4 * e + 3][i] + nan_or_0);
          if (q4 == 0) a.part_ml[sidx] = make_float2(m_ref, l);
        }
      }
    }
    if (!has_next) break;
    ++round;
    nx = nx2;
    cur = nxt;
    btv = btv_next;
    btv_bad = btv_next_bad;
  }
}

// Persistent grid: as many 4-wave workgroups as fit on the device at once
// (at most per_cu per CU), but no more than the work items need.
// (One cached occupancy per kernel: the template argument is the kernel.  The
// cache is the library's only process-wide state: written once per kernel
// with the value the runtime reports, which is the same for every caller, so
// concurrent first calls race benignly.)
template <auto K>
int64_t persistent_grid(int64_t bound_wgs, int cus, int per_cu = 64) {
  static std::atomic<int> occ_cache{0};
  int occ = occ_cache.load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, K, 256, 0) != hipSuccess || occ <= 0)
      occ = 2;
    occ_cache.store(occ, std::memory_order_relaxed);
  }
  return std::max<int64_t>(1, std::min<int64_t>(bound_wgs, (int64_t)cus * std::min(occ, per_cu)));
}

template <bool BF16, int D, int GM>
int launch_rows_g(const RowParams& p, int64_t bound_waves, int cus, hipStream_t s) {
  auto k = row_attn_kernel<BF16, D, GM>;
  // bf16 at head_dim 128: one workgroup (one wave per SIMD) per CU streams
  // as fast as two
  const int64_t grid =
      persistent_grid<row_attn_kernel<BF16, D, GM>>((bound_waves + 3) / 4, cus, BF16 && D == 128 ? 1 : 64);
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool BF16, int D>
int launch_rows_d(const RowParams& p, int64_t bound_waves, int cus, hipStream_t s) {
  // (wider groups arrive split into head_groups of kMaxGroupRegs heads)
  static_assert(kMaxGroupRegs == 4, "instantiations below cover 1, 2 and 4 heads per wave");
  const int gm = p.head_groups > 1 ? kMaxGroupRegs : p.group;
  if (gm <= 1) return launch_rows_g<BF16, D, 1>(p, bound_waves, cus, s);
  if (gm <= 2) return launch_rows_g<BF16, D, 2>(p, bound_waves, cus, s);
  // (bf16 groups of 3 or 4 at head_dim 128 run on the MFMA row kernel)
  if constexpr (!(BF16 && D == 128))
    if (gm <= 4) return launch_rows_g<BF16, D, 4>(p, bound_waves, cus, s);
  return 1;
}

}  // namespace

// bf16 groups wider than kMaxGroupRegs run on row_attn_mfma_kernel, one wave
// for the whole group (as several waves of 4 heads, each reading the blocks,
// they measured 7% slower at G = 8), and so do groups of 3 or 4 at head_dim
// 128 (measured 3-4% faster there than the 4-head VALU kernel, but 2%
// slower at head_dim 64); one- and two-head groups and fp32 run on
// row_attn_kernel, which is as fast or faster there.
bool rows_on_mfma(int32_t dtype, int32_t group, int32_t head_dim) {
  return dtype == PKV_BF16 && (group > kMaxGroupRegs || (group > 2 && head_dim == 128));
}

int max_group_regs(int32_t dtype, int32_t group, int32_t head_dim) {
  return rows_on_mfma(dtype, group, head_dim) ? 16 : kMaxGroupRegs;
}

int launch_rows(const RowParams& p, int32_t dtype, int32_t head_dim, int64_t bound_waves, int cus,
                hipStream_t stream) {
  if (bound_waves <= 0) return 0;
  const bool bf16 = dtype == PKV_BF16;
  if (rows_on_mfma(dtype, p.group, head_dim)) {  // the whole group in one wave (head_groups == 1)
    auto k = head_dim == 64 ? row_attn_mfma_kernel<64> : row_attn_mfma_kernel<128>;
    const int64_t grid = head_dim == 64 ? persistent_grid<row_attn_mfma_kernel<64>>((bound_waves + 3) / 4, cus)
                                        : persistent_grid<row_attn_mfma_kernel<128>>((bound_waves + 3) / 4, cus, 1);
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
  if (head_dim == 64) return bf16 ? launch_rows_d<true, 64>(p, bound_waves, cus, stream)
                                  : launch_rows_d<false, 64>(p, bound_waves, cus, stream);
  return bf16 ? launch_rows_d<true, 128>(p, bound_waves, cus, stream)
              : launch_rows_d<false, 128>(p, bound_waves, cus, stream);
}

}  // namespace pkv
