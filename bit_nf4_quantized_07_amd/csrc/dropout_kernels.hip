// LoRA dropout on the adapter input.  Every training recipe on the pages sets
// lora_dropout = 0.05 (aigrafen.se "QLoRA", code block; llm-compass "QLoRA",
// code under 实现要点; skillbyai "A QLoRA setup in outline";
// learn-interview-questions §3): the input of the down projection A is
// dropped elementwise and rescaled by 1 / (1 - p), the frozen base sees the
// undropped input.
//
// The random words come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-based
// generator: element i of the row-major [M, K] input uses word i % 4 of the
// block for counter (g mod 2^32, g div 2^32, 0, 0), g = i div 4, under the
// 64-bit seed as key, so every element's draw is a pure function of
// (seed, i) and any kernel can regenerate or check it.  Element i is kept
// when its word is >= floor(p 2^32) (computed on the host).
#include "device_common.h"
#include "kernels.h"

namespace qlk {

// One Philox4x32 block: ten rounds of two 32 x 32 -> 64-bit products with the
// published multipliers, the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                   (uint32_t)p0);
  }
  return c;
}

// One thread per 32 consecutive elements (one mask word): eight Philox
// blocks, four 16-byte loads and stores of the bf16 data.  Kept elements are
// bf16(fp32(x * scale)) with round to nearest even, dropped ones +0.
__global__ void __launch_bounds__(256)
k_lora_dropout(const uint16_t* __restrict__ X, int64_t nwords, uint32_t threshold, float scale,
               uint32_t k0, uint32_t k1, uint16_t* __restrict__ Xd, uint32_t* __restrict__ mask) {
  const int64_t wd = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wd >= nwords) return;
  const uint4* src = reinterpret_cast<const uint4*>(X) + wd * 4;
  uint4* dst = reinterpret_cast<uint4*>(Xd) + wd * 4;
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {               // 8 elements per 16-byte piece
    const uint4 xv = src[q];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t o[4];
#pragma unroll
    for (int hblk = 0; hblk < 2; ++hblk) {    // two Philox blocks per piece
      const uint64_t g = (uint64_t)wd * 8 + 2 * q + hblk;
      const uint4 rw = philox4x32_10(make_uint4((uint32_t)g, (uint32_t)(g >> 32), 0u, 0u), k0, k1);
      const uint32_t r4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {           // two bf16 per 32-bit word
        const uint32_t wv = xw[2 * hblk + e];
        float v[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bool keep = r4[2 * e + j] >= threshold;
          const float x = bf16_to_f32(j ? (wv >> 16) : (wv & 0xffffu));
          v[j] = keep ? x * scale : 0.0f;
          bits |= (keep ? 1u : 0u) << (8 * q + 4 * hblk + 2 * e + j);
        }
        o[2 * hblk + e] = pack_bf16x2(v[0], v[1]);
      }
    }
    dst[q] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  mask[wd] = bits;
}

hipError_t launch_lora_dropout(const uint16_t* X, int64_t numel, uint32_t threshold, float scale,
                               uint64_t seed, uint16_t* Xd, uint32_t* mask, hipStream_t st) {
  const int64_t nwords = numel / 32;
  hipLaunchKernelGGL(k_lora_dropout, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, st, X,
                     nwords, threshold, scale, (uint32_t)seed, (uint32_t)(seed >> 32), Xd, mask);
  return hipGetLastError();
}

// dX[m, k] (+)= bf16(mask(m, k) keep_scale sum_j U[m, j] (s A[j, k])), the
// masked adapter term alone.  One thread per 8 consecutive k of one row m;
// (s A) is rounded to bf16 as in the fused dX kernel, the sum over j runs in
// order in fp32.
__global__ void __launch_bounds__(256)
k_dx_adapter_masked(const uint16_t* __restrict__ U, const uint16_t* __restrict__ A, int64_t M,
                    int64_t K, int r, float s, const uint32_t* __restrict__ mask, float keep_scale,
                    uint16_t* __restrict__ dX, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = K / 8;
  if (t >= M * per_row) return;
  const int64_t m = t / per_row, k = (t % per_row) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < r; ++j) {
    const float u = bf16_to_f32(U[m * r + j]);
    const uint4 av = *reinterpret_cast<const uint4*>(A + (int64_t)j * K + k);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_to_f32(f32_to_bf16(bf16_to_f32(aw[e] & 0xffffu) * s));
      const float hi = bf16_to_f32(f32_to_bf16(bf16_to_f32(aw[e] >> 16) * s));
      acc[2 * e] = __builtin_fmaf(u, lo, acc[2 * e]);
      acc[2 * e + 1] = __builtin_fmaf(u, hi, acc[2 * e + 1]);
    }
  }
  const int64_t i0 = m * K + k;                 // 8 consecutive bits of one word (K % 8 == 0)
  const uint32_t bits = (mask[i0 >> 5] >> (i0 & 31)) & 0xffu;
  uint4* dst = reinterpret_cast<uint4*>(dX + i0);
  uint4 old = make_uint4(0, 0, 0, 0);
  if (accumulate) old = *dst;
  const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v0 = ((bits >> (2 * e)) & 1u) ? acc[2 * e] * keep_scale : 0.0f;
    float v1 = ((bits >> (2 * e + 1)) & 1u) ? acc[2 * e + 1] * keep_scale : 0.0f;
    if (accumulate) {
      v0 += bf16_to_f32(ow[e] & 0xffffu);
      v1 += bf16_to_f32(ow[e] >> 16);
    }
    o[e] = pack_bf16x2(v0, v1);
  }
  *dst = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_dx_adapter_masked(const uint16_t* U, const uint16_t* A, int64_t M, int64_t K,
                                    int r, float s, const uint32_t* mask, float keep_scale,
                                    uint16_t* dX, bool accumulate, hipStream_t st) {
  const int64_t threads = M * (K / 8);
  hipLaunchKernelGGL(k_dx_adapter_masked, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     U, A, M, K, r, s, mask, keep_scale, dX, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace qlk
