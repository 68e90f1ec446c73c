// Staging of an 8-bit cache's prefill blocks: each cache block that the
// step's prefill chunks read is dequantised once into a bf16 block of the
// staging area, which the bf16 prefill kernel then reads through the staging
// block table the plan wrote.  (Dequantising inside the prefill kernel instead
// costs the same conversion once per prefill tile that reads the block, i.e.
// once per query tile of the request and kv head.)
//
// The dequantised value is the code times its row's scale in float32, rounded
// to bf16 to nearest even: the values the prefill kernel's in-LDS
// dequantisation forms ("KV Cache 量化", lpnh.cn/news/2436702 section 4.2:
// an 8-bit code and a per-row scale), so staging does not change a result bit.
// INT8 codes are two's complement bytes; FP8 codes are OCP E4M3 (every E4M3
// value is a float32 value, so its conversion is exact).
#include "pkv_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

PKV_DEV uint32_t pack_bf16_rne(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// One workgroup per staged block and half (K or V) at a time; a thread turns
// 16 codes (one 16-byte load) of one token row of one kv head into 32 bytes
// of bf16, for up to kPer chunks whose loads are all issued before the first
// store.  Codes: [2][num_blocks][16][Hkv][D] bytes; scales: [2][num_blocks]
// [Hkv][16] floats; staged: [2][capacity][16][Hkv][D] bf16.
constexpr int kStageThreads = 256;
constexpr int kPer = 4;   // chunks per thread per pass: a half block at Hkv * D = 1024

template <bool FP8>
__global__ __launch_bounds__(kStageThreads) void stage_kernel(StageParams a, const uint8_t* __restrict__ cache,
                                                               const float* __restrict__ kv_scales,
                                                               uint16_t* __restrict__ staged) {
  const int64_t total = a.hdr[kHdrStagedBlocks];
  const int Hkv = a.num_kv_heads, D = a.head_dim;
  const int chunks = kBlock * Hkv * D / 16;          // 16-code chunks of one half block
  const int64_t units = 2 * total;                   // (staged block, half)
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t sb = u >> 1;
    const int kv = (int)(u & 1);
    const int64_t src = a.src[sb];
    const uint8_t* codes = cache + ((size_t)kv * a.num_blocks + src) * kBlock * Hkv * D;
    const float* scales = kv_scales + ((size_t)kv * a.num_blocks + src) * Hkv * kBlock;
    uint32_t* dst = (uint32_t*)(staged + ((size_t)kv * a.capacity + sb) * kBlock * Hkv * D);
    for (int c0 = threadIdx.x; c0 < chunks; c0 += kPer * kStageThreads) {
      u32x4 cw[kPer];
      float sc[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = (c0 + j * kStageThreads) * 16;  // first code of the chunk
        const int row = e / (Hkv * D);                // token row of the block
        const int h = (e - row * Hkv * D) / D;        // kv head
        if (c0 + j * kStageThreads < chunks) {
          cw[j] = *(const u32x4*)(codes + e);
          sc[j] = scales[h * kBlock + row];
        }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (c0 + j * kStageThreads >= chunks) break;
        const int e = (c0 + j * kStageThreads) * 16;
        uint32_t o[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if constexpr (FP8) {
            float f[4];
            fp8x4(cw[j][d], f);
            o[2 * d] = pack_bf16_rne(f[0] * sc[j], f[1] * sc[j]);
            o[2 * d + 1] = pack_bf16_rne(f[2] * sc[j], f[3] * sc[j]);
          } else {
            const int x = (int)cw[j][d];
            o[2 * d] = pack_bf16_rne((float)((x << 24) >> 24) * sc[j], (float)((x << 16) >> 24) * sc[j]);
            o[2 * d + 1] = pack_bf16_rne((float)((x << 8) >> 24) * sc[j], (float)(x >> 24) * sc[j]);
          }
        }
        *(u32x4*)(dst + e / 2) = u32x4{o[0], o[1], o[2], o[3]};
        *(u32x4*)(dst + e / 2 + 4) = u32x4{o[4], o[5], o[6], o[7]};
      }
    }
  }
}

}  // namespace

int launch_stage(const StageParams& p, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return 0;
  auto k = p.fp8 ? stage_kernel<true> : stage_kernel<false>;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kStageThreads), 0, stream, p, (const uint8_t*)p.cache, p.kv_scales,
                     (uint16_t*)p.staged);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace pkv
