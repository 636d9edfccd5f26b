// Gated-MLP glue used by the MLP workloads: H = silu(G) * Up and its
// derivative, bf16 in and out, fp32 inside.  Not a QLoRA step; the pages only
// name gate/up/down projections as adapter targets.
#include "device_common.h"
#include "kernels.h"

namespace qlk {


__global__ void __launch_bounds__(256)
k_silu_mul_fwd(const uint16_t* __restrict__ G, const uint16_t* __restrict__ U, int64_t n8,
               uint16_t* __restrict__ H) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint4 gv = reinterpret_cast<const uint4*>(G)[i];
  const uint4 uv = reinterpret_cast<const uint4*>(U)[i];
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float g0 = bf16_to_f32(gw[q] & 0xffffu), g1 = bf16_to_f32(gw[q] >> 16);
    const float u0 = bf16_to_f32(uw[q] & 0xffffu), u1 = bf16_to_f32(uw[q] >> 16);
    o[q] = pack_bf16x2(silu_mul_f32(g0, u0), silu_mul_f32(g1, u1));
  }
  reinterpret_cast<uint4*>(H)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ void __launch_bounds__(256)
k_silu_mul_bwd(const uint16_t* __restrict__ dH, const uint16_t* __restrict__ G,
               const uint16_t* __restrict__ U, int64_t n8, uint16_t* __restrict__ dG,
               uint16_t* __restrict__ dU) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint4 hv = reinterpret_cast<const uint4*>(dH)[i];
  const uint4 gv = reinterpret_cast<const uint4*>(G)[i];
  const uint4 uv = reinterpret_cast<const uint4*>(U)[i];
  const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w},
                 uw[4] = {uv.x, uv.y, uv.z, uv.w};
  uint32_t og[4], ou[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float rg[2], ru[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float d = bf16_to_f32(h ? hw[q] >> 16 : hw[q] & 0xffffu);
      const float g = bf16_to_f32(h ? gw[q] >> 16 : gw[q] & 0xffffu);
      const float u = bf16_to_f32(h ? uw[q] >> 16 : uw[q] & 0xffffu);
      const float sg = sigmoidf_(g);
      rg[h] = d * u * sg * (1.0f + g * (1.0f - sg));
      ru[h] = d * g * sg;
    }
    og[q] = pack_bf16x2(rg[0], rg[1]);
    ou[q] = pack_bf16x2(ru[0], ru[1]);
  }
  reinterpret_cast<uint4*>(dG)[i] = make_uint4(og[0], og[1], og[2], og[3]);
  reinterpret_cast<uint4*>(dU)[i] = make_uint4(ou[0], ou[1], ou[2], ou[3]);
}

hipError_t launch_silu_mul_fwd(const uint16_t* G, const uint16_t* U, int64_t n, uint16_t* H,
                               hipStream_t st) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_silu_mul_fwd, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, G, U, n8, H);
  return hipGetLastError();
}

hipError_t launch_silu_mul_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* U,
                               int64_t n, uint16_t* dG, uint16_t* dU, hipStream_t st) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_silu_mul_bwd, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, dH, G, U,
                     n8, dG, dU);
  return hipGetLastError();
}

// dst [rows_dst, cols_dst] = src [rows_src, cols_src] zero-extended (or cut)
// to the new shape, both row-major and contiguous.  The adapter rank is
// padded with it to the kernels' granule (zero rows of A, zero columns of B
// and T) and the results are cut back to the caller's rank.
template <class T>
__global__ void __launch_bounds__(256)
k_pad2d(const T* __restrict__ src, int64_t rows_src, int64_t cols_src, T* __restrict__ dst,
        int64_t rows_dst, int64_t cols_dst) {
  const int64_t n = rows_dst * cols_dst;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / cols_dst, col = i - row * cols_dst;
    dst[i] = (row < rows_src && col < cols_src) ? src[row * cols_src + col] : T(0);
  }
}

template <class T>
static hipError_t pad2d(const T* src, int64_t rows_src, int64_t cols_src, T* dst, int64_t rows_dst,
                        int64_t cols_dst, hipStream_t st) {
  const int64_t n = rows_dst * cols_dst;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(k_pad2d<T>, dim3((unsigned)blocks), dim3(256), 0, st, src, rows_src, cols_src,
                     dst, rows_dst, cols_dst);
  return hipGetLastError();
}

hipError_t launch_pad2d(const uint16_t* src, int64_t rows_src, int64_t cols_src, uint16_t* dst,
                        int64_t rows_dst, int64_t cols_dst, hipStream_t st) {
  return pad2d(src, rows_src, cols_src, dst, rows_dst, cols_dst, st);
}

hipError_t launch_pad2d(const float* src, int64_t rows_src, int64_t cols_src, float* dst,
                        int64_t rows_dst, int64_t cols_dst, hipStream_t st) {
  return pad2d(src, rows_src, cols_src, dst, rows_dst, cols_dst, st);
}

}  // namespace qlk
