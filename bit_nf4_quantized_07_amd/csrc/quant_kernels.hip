// Bit-exact storage kernels: NF4 blockwise quantisation, double quantisation
// of the block constants, and dequantisation to bf16.
//
// Format (aigrafen.se "QLoRA", list "Tre tekniska bitar" items 1-2;
// llm-compass "QLoRA", 方法与公式 items 1-2): 4-bit NormalFloat codes in
// blocks of 64 consecutive weights with one absmax constant each; the
// constants are quantised again to 8 bits around their mean with one fp32
// scale per 256 constants.
#include <math.h>
#include <string.h>

#include "device_common.h"
#include "kernels.h"
#include "dequant_block.h"

namespace qlk {

// ---------------------------------------------------------------------------
// nf4_quantize: 8 lanes per block of 64, each lane 8 consecutive weights.
// ---------------------------------------------------------------------------
// The codebook (NF4, or another 16-level table such as uniform INT4) comes
// in as a kernel argument with its decision thresholds.
__global__ void __launch_bounds__(256)
k_nf4_quantize(const float* __restrict__ W, int64_t nblocks, Codebook4 cb,
               uint8_t* __restrict__ packed, float* __restrict__ absmax) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  // Whole groups of 8 lanes are in or out together (nblocks*8 threads).
  if (blk >= nblocks) return;

  float thr[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) thr[i] = cb.thr[i];

  const float4* src = reinterpret_cast<const float4*>(W + blk * kBlock + sub * 8);
  const float4 a = src[0], b = src[1];
  float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(w[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 4, 8));

  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // IEEE division (correctly rounded); an all-zero block has n = 0 (the
    // NF4 zero level, index 7).
    const float n = (m > 0.0f) ? w[i] / m : 0.0f;
    // The number of thresholds strictly below n, by a binary search over the
    // ascending thresholds (the same count as comparing with all 15): each
    // step picks the threshold to compare with by selects, no indexing.
    uint32_t c = n > thr[7] ? 8u : 0u;
    {
      const float t4 = c ? thr[11] : thr[3];
      c += n > t4 ? 4u : 0u;
      const float t2 = (c & 8u) ? ((c & 4u) ? thr[13] : thr[9]) : ((c & 4u) ? thr[5] : thr[1]);
      c += n > t2 ? 2u : 0u;
      const float ta = (c & 2u) ? ((c & 4u) ? thr[6] : thr[2]) : ((c & 4u) ? thr[4] : thr[0]);
      const float tb = (c & 2u) ? ((c & 4u) ? thr[14] : thr[10]) : ((c & 4u) ? thr[12] : thr[8]);
      c += n > ((c & 8u) ? tb : ta) ? 1u : 0u;
    }
    // element 2j -> high nibble of byte j; bytes little-endian in the word
    const int byte = i >> 1;
    const int shift = byte * 8 + ((i & 1) ? 0 : 4);
    word |= c << shift;
  }
  reinterpret_cast<uint32_t*>(packed + blk * (kBlock / 2))[sub] = word;
  if (sub == 0) absmax[blk] = m;
}

// ---------------------------------------------------------------------------
// double_quant, step 1: the per-tensor mean in a fixed summation order.
// One workgroup of 1024 lanes.  Lane t sums constant-group (base + t)
// sequentially in fp64; lane 0 then adds the group sums sequentially.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024)
k_dq_mean(const float* __restrict__ absmax, int64_t nb, float* __restrict__ mean) {
  __shared__ double part[1024];
  const int64_t ngroups = (nb + kDQBlock - 1) / kDQBlock;
  double total = 0.0;
  for (int64_t base = 0; base < ngroups; base += 1024) {
    const int64_t g = base + threadIdx.x;
    if (g < ngroups) {
      const int64_t lo = g * kDQBlock;
      const int64_t hi = (lo + kDQBlock < nb) ? lo + kDQBlock : nb;
      double s = 0.0;
      for (int64_t i = lo; i < hi; ++i) s += (double)absmax[i];
      part[threadIdx.x] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int64_t lim = (ngroups - base < 1024) ? ngroups - base : 1024;
      for (int64_t j = 0; j < lim; ++j) total += part[j];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = (float)(total / (double)nb);
}

// double_quant, step 1 for more than one group, in two launches with the same
// summation order: (a) one thread per group of 256 constants forms the
// group's sequential fp64 sum; (b) one workgroup stages the group sums in LDS
// and one thread adds them in index order.  The group sums live in the codes
// buffer until step 2 overwrites it (8 bytes per group, 256 code bytes).
__global__ void __launch_bounds__(64)
k_dq_group_sums(const float* __restrict__ absmax, int64_t nb, double* __restrict__ sums) {
  const int64_t ngroups = (nb + kDQBlock - 1) / kDQBlock;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ngroups) return;
  const int64_t lo = g * kDQBlock;
  const int64_t hi = (lo + kDQBlock < nb) ? lo + kDQBlock : nb;
  double s = 0.0;
  if (hi - lo == kDQBlock) {
    // a whole group: all 64 loads in flight, then the ordered additions
    const float4* p = reinterpret_cast<const float4*>(absmax + lo);
#pragma unroll 16
    for (int i = 0; i < kDQBlock / 4; ++i) {
      const float4 v = p[i];
      s += (double)v.x; s += (double)v.y; s += (double)v.z; s += (double)v.w;
    }
  } else {
    for (int64_t i = lo; i < hi; ++i) s += (double)absmax[i];
  }
  sums[g] = s;
}

constexpr int kDqChunk = 4096;   // group sums staged in LDS per round (32 KB)

__global__ void __launch_bounds__(256)
k_dq_mean_ordered(const double* __restrict__ sums, int64_t ngroups, int64_t nb,
                  float* __restrict__ mean) {
  __shared__ double part[kDqChunk];
  double total = 0.0;
  for (int64_t base = 0; base < ngroups; base += kDqChunk) {
    const int64_t n = (ngroups - base < kDqChunk) ? ngroups - base : kDqChunk;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) part[i] = sums[base + i];
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll 16
      for (int64_t j = 0; j < n; ++j) total += part[j];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = (float)(total / (double)nb);
}

// ---------------------------------------------------------------------------
// double_quant, step 2: one workgroup per group of 256 constants.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_dq_codes(const float* __restrict__ absmax, int64_t nb, const float* __restrict__ mean,
           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float thr[254];
  __shared__ float wmax[4];
  for (int i = threadIdx.x; i < 254; i += blockDim.x) thr[i] = dq_threshold(i);

  const int64_t i = (int64_t)blockIdx.x * kDQBlock + threadIdx.x;
  const bool valid = i < nb;
  const float mu = mean[0];
  const float c = valid ? absmax[i] - mu : 0.0f;
  float m = fabsf(c);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float s = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  const float n2 = (s > 0.0f) ? c / s : 0.0f;
  // code = number of thresholds strictly below n2 (binary search).
  int lo = 0, hi = 254;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (n2 > thr[mid]) lo = mid + 1; else hi = mid;
  }
  if (valid) codes[i] = (uint8_t)lo;
  if (threadIdx.x == 0) scales[blockIdx.x] = s;
}

// double_quant with a second-level table passed as data (the same rules: the
// code is the number of thresholds strictly below fp32(c / s_g), so ties go
// to the lower index and a group with s_g = 0 gets the index of the level
// nearest zero).
__global__ void __launch_bounds__(256)
k_dq_codes_table(const float* __restrict__ absmax, int64_t nb, const float* __restrict__ mean,
                 Codebook8 cb, uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float thr[255];
  __shared__ float wmax[4];
  const int nthr = cb.n - 1;
  for (int i = threadIdx.x; i < nthr; i += blockDim.x) thr[i] = cb.thr[i];

  const int64_t i = (int64_t)blockIdx.x * kDQBlock + threadIdx.x;
  const bool valid = i < nb;
  const float mu = mean[0];
  const float c = valid ? absmax[i] - mu : 0.0f;
  float m = fabsf(c);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float s = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float n2 = (s > 0.0f) ? c / s : 0.0f;
  int lo = 0, hi = nthr;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (n2 > thr[mid]) lo = mid + 1; else hi = mid;
  }
  if (valid) codes[i] = (uint8_t)lo;
  if (threadIdx.x == 0) scales[blockIdx.x] = s;
}

// a_hat of every block: fp32(fp32(levels[code] * s_g) + mean), one thread per
// block, the table staged in LDS (codes past the table's end read 0).
__global__ void __launch_bounds__(256)
k_absmax_dequant(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                 const float* __restrict__ mean, int64_t nb, Codebook8 cb, float* __restrict__ out) {
  __shared__ float q8[256];
  q8[threadIdx.x] = cb.lv[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nb) return;
  out[i] = absmax_decode_tab((int)codes[i], scales[i / kDQBlock], mean[0], q8);
}

// ---------------------------------------------------------------------------
// nf4_dequant: a wave expands 2048 consecutive weights (1 KB packed, 4 KB
// out) in four rounds; in round q lane L turns packed word 64 q + L (8
// weights) into 16 bytes at output offset 1 KB q + 16 L, so every load and
// every store instruction of the wave covers one contiguous range.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_nf4_dequant(const uint8_t* __restrict__ packed, const uint8_t* __restrict__ codes,
              const float* __restrict__ scales, const float* __restrict__ mean,
              int64_t nwords, Codebook4 cb, uint16_t* __restrict__ out) {
  nf4_dequant_block(packed, codes, scales, mean, nwords, cb, out, blockIdx.x);
}

// The same with the 8-bit levels from a table (staged in LDS).
__global__ void __launch_bounds__(256)
k_dequant_tables(const uint8_t* __restrict__ packed, const uint8_t* __restrict__ codes,
                 const float* __restrict__ scales, const float* __restrict__ mean, int64_t nwords,
                 Codebook4 cb, Codebook8 cb8, uint16_t* __restrict__ out) {
  __shared__ float q8[256];
  q8[threadIdx.x] = cb8.lv[threadIdx.x];
  __syncthreads();
  nf4_dequant_block(packed, codes, scales, mean, nwords, cb, out, blockIdx.x, q8);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
Codebook4 make_codebook(const float* levels16) {
  Codebook4 cb;
  for (int i = 0; i < 16; ++i) cb.lv[i] = levels16[i];
  for (int i = 0; i < 15; ++i) {
    const double m = ((double)cb.lv[i] + (double)cb.lv[i + 1]) * 0.5;   // exact in fp64
    float t = (float)m;
    if ((double)t > m) t = nextafterf(t, -INFINITY);                    // round toward -inf
    cb.thr[i] = t;
  }
  return cb;
}

Codebook8 make_codebook8(const float* levels, int n) {
  Codebook8 cb;
  cb.n = n;
  for (int i = 0; i < 256; ++i) cb.lv[i] = i < n ? levels[i] : 0.0f;
  for (int i = 0; i < 255; ++i) {
    cb.thr[i] = 0.0f;
    if (i + 1 >= n) continue;
    const double m = ((double)cb.lv[i] + (double)cb.lv[i + 1]) * 0.5;   // exact in fp64
    float t = (float)m;
    if ((double)t > m) t = nextafterf(t, -INFINITY);                    // round toward -inf
    cb.thr[i] = t;
  }
  return cb;
}

Codebook4 nf4_codebook4() {
  float lv[16];
  for (int i = 0; i < 16; ++i) memcpy(&lv[i], &kNF4Bits[i], 4);
  return make_codebook(lv);
}

hipError_t launch_nf4_quantize(const float* W, int64_t numel, const Codebook4& cb, uint8_t* packed,
                               float* absmax, hipStream_t st) {
  const int64_t nb = numel / kBlock;
  const int64_t threads = nb * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(k_nf4_quantize, dim3((unsigned)grid), dim3(256), 0, st, W, nb, cb, packed,
                     absmax);
  return hipGetLastError();
}

hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* codes, float* scales,
                               float* mean, hipStream_t st, const Codebook8* cb8) {
  const int64_t ng = (nb + kDQBlock - 1) / kDQBlock;
  if (ng == 1) {
    hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(1024), 0, st, absmax, nb, mean);
  } else {
    // ng >= 2 groups: nb > 256 (ng - 1) >= 8 ng, so the codes buffer (nb
    // bytes, 16-byte aligned) holds the ng fp64 group sums.
    double* sums = reinterpret_cast<double*>(codes);
    hipLaunchKernelGGL(k_dq_group_sums, dim3((unsigned)((ng + 63) / 64)), dim3(64), 0, st, absmax,
                       nb, sums);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
    hipLaunchKernelGGL(k_dq_mean_ordered, dim3(1), dim3(256), 0, st, sums, ng, nb, mean);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (cb8)
    hipLaunchKernelGGL(k_dq_codes_table, dim3((unsigned)ng), dim3(256), 0, st, absmax, nb, mean,
                       *cb8, codes, scales);
  else
    hipLaunchKernelGGL(k_dq_codes, dim3((unsigned)ng), dim3(256), 0, st, absmax, nb, mean, codes,
                       scales);
  return hipGetLastError();
}

hipError_t launch_absmax_dequant(const uint8_t* codes, const float* scales, const float* mean,
                                 int64_t nb, const Codebook8& cb8, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_absmax_dequant, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, codes,
                     scales, mean, nb, cb8, out);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                              const float* mean, int64_t numel, const Codebook4& cb, uint16_t* out,
                              hipStream_t st, const Codebook8* cb8) {
  const int64_t nwords = numel / 8;                  // numel % 64 == 0
  const int64_t grid = (nwords + 4 * kDqWaveWords - 1) / (4 * kDqWaveWords);   // 4 waves
  if (cb8)
    hipLaunchKernelGGL(k_dequant_tables, dim3((unsigned)grid), dim3(256), 0, st, packed, codes,
                       scales, mean, nwords, cb, *cb8, out);
  else
    hipLaunchKernelGGL(k_nf4_dequant, dim3((unsigned)grid), dim3(256), 0, st, packed, codes,
                       scales, mean, nwords, cb, out);
  return hipGetLastError();
}

}  // namespace qlk
