// paged_kv_write: store each new token's K and V rows at its slot.
//
// "AI Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention":
// slot_mapping tells the kernel which slot a new token's K/V goes to, and a
// slot names block slot / block_size, offset slot % block_size.  Inside a
// block the layout is [block_size][num_kv_heads][head_dim], so the slot
// index, taken as a row number of the [num_blocks * 16] row array of one
// half (K or V), addresses the token's whole [num_kv_heads][head_dim] row.
//
// One thread moves one 16-byte chunk; consecutive threads move consecutive
// chunks of a token row, so both the read of k/v and the write into the
// cache are fully coalesced.  The copy is bit-exact.
#include <algorithm>

#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, u32x4* __restrict__ cache,
    int64_t num_tokens, int64_t num_slots, int32_t chunks_per_row,
    int32_t* __restrict__ device_error) {
  const int64_t per_token = 2 * (int64_t)chunks_per_row;
  const int64_t total = num_tokens * per_token;
  const int64_t half = num_slots * chunks_per_row;  // chunks in the K half
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int32_t rem = (int32_t)(i - t * per_token);
    const int32_t kv = rem >= chunks_per_row;
    const int32_t ch = rem - kv * chunks_per_row;
    const int64_t slot = slot_mapping[t];
    if (slot == -1) continue;  // padding token
    if (slot < 0 || slot >= num_slots) {
      if (device_error != nullptr && ch == 0 && kv == 0) atomicOr(device_error, PKV_DEVERR_SLOT);
      continue;
    }
    const u32x4* src = kv ? v : k;
    cache[kv * half + slot * chunks_per_row + ch] = src[t * chunks_per_row + ch];
  }
}

int launch_kv_write(const void* k, const void* v, const int64_t* slot_mapping, void* cache,
                    int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, int32_t elem_bytes, int32_t* device_error,
                    hipStream_t stream) {
  if (num_tokens == 0) return 0;
  const int32_t chunks = num_kv_heads * head_dim * elem_bytes / 16;
  const int64_t total = num_tokens * 2 * chunks;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const u32x4*)k, (const u32x4*)v, slot_mapping, (u32x4*)cache,
                     num_tokens, (int64_t)num_blocks * kBlock, chunks, device_error);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// paged_kv_write_rope: the same scatter with the rotary position embedding
// applied to K on the way ("AI Infra入门干货总结", section "LLM 推理全流程" /
// "RoPE": positions are rotation angles read from a precomputed
// cos_sin_cache [max_position, rotary_dim]; row p = cos of the rotary_dim/2
// angles of position p, then their sin).  Angle i rotates the pair
// (i, i + rotary_dim/2) when is_neox, else (2i, 2i+1):
// x' = x cos - y sin, y' = y cos + x sin, in fp32, rounded to the storage
// type; dims from rotary_dim on and all of V are copied unchanged.  When q is
// given, its rows are rotated in place the same way, so one launch does the
// step's whole rotary work.  One workgroup per token (grid-stride): the
// token's cos/sin row is read once; consecutive threads take consecutive
// pairs (neox: both halves are contiguous runs; interleaved: adjacent
// elements), so every access is coalesced.
template <bool BF16>
struct RopeElem;
template <>
struct RopeElem<true> {
  using T = uint16_t;
  PKV_DEV static float ld(const T* p) { return __uint_as_float((uint32_t)*p << 16); }
  PKV_DEV static void st(T* p, float x) { *p = f32_to_bf16(x); }
};
template <>
struct RopeElem<false> {
  using T = float;
  PKV_DEV static float ld(const T* p) { return *p; }
  PKV_DEV static void st(T* p, float x) { *p = x; }
};

template <bool BF16>
PKV_DEV void rope_rows(const typename RopeElem<BF16>::T* src, typename RopeElem<BF16>::T* dst, int heads,
                       int head_dim, int half, bool neox, const float* cs) {
  using E = RopeElem<BF16>;
  for (int u = threadIdx.x; u < heads * half; u += blockDim.x) {
    const int h = u / half, i = u - h * half;
    const int ix = neox ? i : 2 * i, iy = neox ? i + half : 2 * i + 1;
    const float c = cs[i], s = cs[half + i];
    const float x = E::ld(src + h * head_dim + ix), y = E::ld(src + h * head_dim + iy);
    E::st(dst + h * head_dim + ix, x * c - y * s);
    E::st(dst + h * head_dim + iy, y * c + x * s);
  }
  const int pass = head_dim - 2 * half;  // dims past rotary_dim
  if (pass > 0 && src != dst)
    for (int u = threadIdx.x; u < heads * pass; u += blockDim.x) {
      const int h = u / pass, e = 2 * half + (u - h * pass);
      dst[h * head_dim + e] = src[h * head_dim + e];
    }
}

template <bool BF16>
__global__ __launch_bounds__(256) void kv_write_rope_kernel(RopeParams a) {
  using T = typename RopeElem<BF16>::T;
  const int half = a.rotary_dim / 2;
  const int64_t num_slots = (int64_t)a.num_blocks * kBlock;
  const int row = a.num_kv_heads * a.head_dim;           // elements of a token's K (or V) row
  const int vchunks = row * (int)sizeof(T) / 16;
  for (int64_t t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
    const int64_t pos = a.positions[t];
    if (pos < 0 || pos >= a.max_position) {  // nothing of this token is touched
      if (threadIdx.x == 0 && a.device_error != nullptr) atomicOr(a.device_error, PKV_DEVERR_POSITION);
      continue;
    }
    const float* cs = a.cos_sin_cache + pos * a.rotary_dim;
    if (a.q != nullptr) {
      T* qrow = (T*)a.q + t * (int64_t)a.num_q_heads * a.head_dim;
      rope_rows<BF16>(qrow, qrow, a.num_q_heads, a.head_dim, half, a.is_neox, cs);
    }
    const int64_t slot = a.slot_mapping[t];
    if (slot == -1) continue;  // padding token: no cache write
    if (slot < 0 || slot >= num_slots) {
      if (threadIdx.x == 0 && a.device_error != nullptr) atomicOr(a.device_error, PKV_DEVERR_SLOT);
      continue;
    }
    T* kc = (T*)a.cache + slot * row;
    rope_rows<BF16>((const T*)a.k + t * row, kc, a.num_kv_heads, a.head_dim, half, a.is_neox, cs);
    const u32x4* vs = (const u32x4*)((const T*)a.v + t * row);
    u32x4* vd = (u32x4*)((T*)a.cache + (num_slots + slot) * row);
    for (int i = threadIdx.x; i < vchunks; i += blockDim.x) vd[i] = vs[i];
  }
}

int launch_kv_write_rope(const RopeParams& p, bool bf16, hipStream_t stream) {
  if (p.num_tokens == 0) return 0;
  const int64_t grid = p.num_tokens < 65536 ? p.num_tokens : 65536;
  if (bf16)
    hipLaunchKernelGGL(kv_write_rope_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_write_rope_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// E4M3 code of a float32 y (OCP 8-bit floating point: bias 7, 3 mantissa
// bits, subnormals m/8 * 2^-6, no infinities, largest finite 448): the
// nearest E4M3 value to y, magnitude clipped at 448, ties to the even code,
// sign bit from y.  Below 2^-6 the steps are 2^-9, so the code is
// round-half-even(|y| * 2^9) (an exact product); above, the float32
// mantissa is rounded to 3 bits half to even, and a carry moves into the
// exponent field by the addition.  448 has code 0x7e and nothing rounds past
// it after the clip, so the NaN code 0x7f never appears.
PKV_DEV uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t e = (b >> 23) - 127u + 7u;
    const uint32_t mant = b & 0x7fffffu;
    uint32_t r = mant >> 20;
    const uint32_t rem = mant & 0xfffffu;
    r += (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
    code = (e << 3) + r;
  }
  return sign | code;
}

// paged_kv_write_int8 / paged_kv_write_fp8: quantise each new token's K and
// V rows, per kv head, to 8-bit codes with one float32 scale, and store both
// at the token's slot (online KV-cache quantisation, lpnh.cn/news/2436702
// section 4.2).  Per (token, K or V, head) row of head_dim values:
//   INT8: scale = max|x| / 127, code = round-half-even(x / scale) clamped to
//         [-127, 127];
//   FP8:  scale = max|x| / 448, code = e4m3_code(x / scale);
// an all-zero row gets scale 0 and codes 0.  Both divisions are IEEE float32
// so the codes are reproducible.  A row is spread over D/8 lanes, 8 values
// each (one 16-byte load of bf16), so a wave holds a set of 64/(D/8) rows;
// wave w of NW takes row sets w, w + NW, ... (up to kI8WPasses of them per
// round) and issues all their loads before the first quantisation.  The row
// max is a reduction over the row's lanes; the row's first lane stores the
// scale.
constexpr int kI8WPasses = 4;

// max over aligned groups of N lanes (N = 8 or 16)
template <int N>
PKV_DEV float group_max(float x) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, N));
  return x;
}

template <bool BF16, int D, bool FP8>
__global__ __launch_bounds__(256) void kv_write_i8_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          int8_t* __restrict__ cache, float* __restrict__ scales,
                                                          int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                                                          int32_t* __restrict__ device_error) {
  constexpr int VPL = 8;               // values per lane
  constexpr int LPR = D / VPL;         // lanes per row
  constexpr int RPW = kWave / LPR;     // rows per wave and pass
  static_assert(LPR == 8 || LPR == 16, "head_dim 64 or 128");
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane / LPR, li = lane % LPR;
  const int64_t rows = num_tokens * 2 * num_kv_heads;
  const int64_t num_slots = (int64_t)num_blocks * kBlock;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int64_t sets = (rows + RPW - 1) / RPW;
  for (int64_t base = wave; base < sets; base += nwaves * kI8WPasses) {
    float x[kI8WPasses][VPL];
    int64_t slot[kI8WPasses];
    int kvh[kI8WPasses];   // kv * num_kv_heads + h
#pragma unroll
    for (int u = 0; u < kI8WPasses; ++u) {
      const int64_t row = (base + u * nwaves) * RPW + sub;
      const bool in = row < rows;
      const int64_t t = in ? row / (2 * num_kv_heads) : 0;
      kvh[u] = in ? (int)(row - t * 2 * num_kv_heads) : 0;
      const int kv = kvh[u] / num_kv_heads, h = kvh[u] - kv * num_kv_heads;
      slot[u] = in ? slot_mapping[t] : -1;
      const size_t src = ((size_t)t * num_kv_heads + h) * D + li * VPL;
      if constexpr (BF16) {
        const u32x4 w = in ? *(const u32x4*)((const uint16_t*)(kv ? v : k) + src) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][2 * e] = __uint_as_float(w[e] << 16);
          x[u][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
        const float* f = (const float*)(kv ? v : k) + src;
        const float4 w0 = in ? *(const float4*)f : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 w1 = in ? *(const float4*)(f + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        x[u][0] = w0.x; x[u][1] = w0.y; x[u][2] = w0.z; x[u][3] = w0.w;
        x[u][4] = w1.x; x[u][5] = w1.y; x[u][6] = w1.z; x[u][7] = w1.w;
      }
    }
#pragma unroll
    for (int u = 0; u < kI8WPasses; ++u) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
      amax = group_max<LPR>(amax);
      const int64_t sl = slot[u];
      if (sl == -1) continue;
      const int kv = kvh[u] / num_kv_heads, h = kvh[u] - kv * num_kv_heads;
      if (sl < 0 || sl >= num_slots) {
        if (device_error != nullptr && li == 0 && kvh[u] == 0) atomicOr(device_error, PKV_DEVERR_SLOT);
        continue;
      }
      const float scale = amax / (FP8 ? 448.f : 127.f);
      uint32_t c[VPL];
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        if constexpr (FP8)
          c[e] = scale > 0.f ? e4m3_code(x[u][e] / scale) : 0u;
        else
          c[e] = scale > 0.f ? (uint32_t)(uint8_t)(int8_t)fminf(fmaxf(rintf(x[u][e] / scale), -127.f), 127.f) : 0u;
      }
      int8_t* dst = cache + ((size_t)kv * num_slots + sl) * num_kv_heads * D + (size_t)h * D + li * VPL;
      *(u32x2*)dst = u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
      // scales [2][num_blocks][num_kv_heads][16]: a head's 16 scales of a block are contiguous
      if (li == 0)
        scales[(((size_t)kv * num_blocks + sl / kBlock) * num_kv_heads + h) * kBlock + sl % kBlock] = scale;
    }
  }
}

int launch_kv_write_i8(const void* k, const void* v, const int64_t* slot_mapping, void* cache, float* scales,
                       int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, bool bf16,
                       bool fp8, int32_t* device_error, hipStream_t stream) {
  if (num_tokens == 0) return 0;
  const int64_t rows = num_tokens * 2 * num_kv_heads;
  // enough waves for kI8WPasses row sets each, and at least 2048 (a round
  // over the whole chip) when there are that many sets
  const int64_t sets = (rows + kWave / (head_dim / 8) - 1) / (kWave / (head_dim / 8));
  const int64_t waves = std::max((sets + kI8WPasses - 1) / kI8WPasses, std::min<int64_t>(sets, 2048));
  int64_t grid = (waves + 3) / 4;   // 4 waves per 256-thread workgroup
  if (grid > 65536) grid = 65536;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream, k, v, slot_mapping, (int8_t*)cache,
                       scales, num_tokens, num_blocks, num_kv_heads, device_error);
  };
  if (fp8) {
    if (head_dim == 64)
      bf16 ? go(kv_write_i8_kernel<true, 64, true>) : go(kv_write_i8_kernel<false, 64, true>);
    else
      bf16 ? go(kv_write_i8_kernel<true, 128, true>) : go(kv_write_i8_kernel<false, 128, true>);
  } else {
    if (head_dim == 64)
      bf16 ? go(kv_write_i8_kernel<true, 64, false>) : go(kv_write_i8_kernel<false, 64, false>);
    else
      bf16 ? go(kv_write_i8_kernel<true, 128, false>) : go(kv_write_i8_kernel<false, 128, false>);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// paged_kv_copy_blocks: destination block <- source block, K and V halves
// (copy-on-write of a shared prefix block, lpnh.cn/news/2436702, section
// 2.2).  A block of one half is 16 * num_kv_heads * head_dim contiguous
// elements, so a pair is two contiguous runs; workgroup (pair, half) copies
// one run with 16-byte chunks, consecutive threads on consecutive chunks.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(u32x4* __restrict__ cache,
                                                             const int32_t* __restrict__ copies,
                                                             int32_t num_copies, int32_t num_blocks,
                                                             int32_t chunks_per_block,
                                                             int32_t* __restrict__ device_error) {
  const int32_t pair = blockIdx.x >> 1;
  const int32_t kv = blockIdx.x & 1;
  if (pair >= num_copies) return;
  const int32_t src = copies[2 * pair], dst = copies[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    if (device_error != nullptr && threadIdx.x == 0 && kv == 0) atomicOr(device_error, PKV_DEVERR_BLOCK_ID);
    return;
  }
  const int64_t half = (int64_t)num_blocks * chunks_per_block;
  const u32x4* s = cache + kv * half + (int64_t)src * chunks_per_block;
  u32x4* d = cache + kv * half + (int64_t)dst * chunks_per_block;
  for (int32_t i = threadIdx.x; i < chunks_per_block; i += blockDim.x) d[i] = s[i];
}

int launch_kv_copy_blocks(void* cache, const int32_t* copies, int32_t num_copies, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes, int32_t* device_error,
                          hipStream_t stream) {
  if (num_copies == 0) return 0;
  const int32_t chunks = kBlock * num_kv_heads * head_dim * elem_bytes / 16;
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3(2u * (unsigned)num_copies), dim3(256), 0, stream,
                     (u32x4*)cache, copies, num_copies, num_blocks, chunks, device_error);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
