// Body of the dequantiser, shared by its own kernel and the backward's
// combined kernel (U = dY B next to the one-off dequantisation).  One wave
// handles 64 kDqRounds packed words in kDqRounds rounds (eight: 512 words,
// 4096 weights, loads of eight words per lane in flight): in round q lane L
// takes word 64 q + L of the wave's range, so every load and store
// instruction of the wave covers one contiguous range.  The block's waves
// take consecutive ranges; `blk` is the block's index in the dequant grid.
// q8: the 8-bit levels as a table in LDS, or null for the linear code.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kDqRounds = 8;                      // rounds per wave (words per lane)
constexpr int kDqWaveWords = 64 * kDqRounds;      // packed words per wave

__device__ __forceinline__ void nf4_dequant_block(const uint8_t* __restrict__ packed,
                                                  const uint8_t* __restrict__ codes,
                                                  const float* __restrict__ scales,
                                                  const float* __restrict__ mean, int64_t nwords,
                                                  const Codebook4& cb, uint16_t* __restrict__ out,
                                                  int64_t blk_index,
                                                  const float* q8 = nullptr) {
  __shared__ float q4[16];
  if (threadIdx.x < 16) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v = (int)threadIdx.x == i ? cb.lv[i] : v;   // no dynamic index
    q4[threadIdx.x] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (blk_index * (blockDim.x >> 6) + (threadIdx.x >> 6)) * kDqWaveWords;  // first word of the wave
  const float mu = mean[0];
  const uint32_t* pw = reinterpret_cast<const uint32_t*>(packed);
  // All rounds' loads first (an out-of-range word loads word 0 and is
  // not stored), so that all of a wave's loads (three per round) are in flight
  // together.
  uint32_t p[kDqRounds], cd[kDqRounds];
  float sc[kDqRounds];
  bool ok[kDqRounds];
#pragma unroll
  for (int q = 0; q < kDqRounds; ++q) {
    const int64_t wd = w0 + 64 * q + lane;   // packed word: weights 8 wd .. 8 wd + 7
    ok[q] = wd < nwords;
    const int64_t wc = ok[q] ? wd : 0;
    const int64_t blk = wc >> 3;             // 8 words per block of 64
    p[q] = pw[wc];
    cd[q] = codes[blk];
    sc[q] = scales[blk / kDQBlock];
  }
#pragma unroll
  for (int q = 0; q < kDqRounds; ++q) {
    if (!ok[q]) continue;
    // 8-bit levels: the linear code computed, or a table (in LDS)
    const float ah = q8 ? absmax_decode_tab((int)cd[q], sc[q], mu, q8) : absmax_decode(cd[q], sc[q], mu);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (p[q] >> (j * 8)) & 0xffu;
      const float a = q4[byte >> 4] * ah;    // element 2j: high nibble
      const float b = q4[byte & 15u] * ah;
      o[j] = pack_bf16x2(a, b);
    }
    reinterpret_cast<uint4*>(out)[w0 + 64 * q + lane] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace qlk
