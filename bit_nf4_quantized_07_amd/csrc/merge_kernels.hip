// Folding the adapter into the dequantised base for serving:
//
//   W_merged = bf16( w_hat + s (B A) ),   s = alpha / r,
//
// with w_hat the bf16 dequantised base weight.  A 4-bit base has to be
// dequantised before the adapter can be merged into it, and the result keeps
// the base's quantisation error (llm-compass "QLoRA", 与 baseline 对比 table,
// row 部署合并, and 实现要点, the item on merging; auryth.ai "QLoRA", FAQ, the
// question on inference; skillbyai "QLoRA: Fine-Tuning on One Consumer GPU",
// "Quantized base plus LoRA").
//
// One workgroup (four waves) owns a 64 (rows n) x 128 (columns k) tile:
//  1. B A for the tile with v_mfma_f32_32x32x16_bf16 in chunks of 16 along r:
//     the operand rows are B's rows (16-byte loads of B [N, r]); the chunk of
//     A [r, K] is staged in LDS and read back with transpose reads, eight
//     consecutive r of one column per lane.  Wave w owns columns 32 w .. +31.
//  2. The fp32 product goes through LDS so that
//  3. each thread then handles four runs of 8 consecutive weights (laid out
//     so that a wave's stores cover whole 256-byte row segments): it decodes
//     them exactly as nf4_dequant does (same bf16 values), adds s (B A) with
//     one fused multiply-add in fp32, rounds to bf16 and stores 16 bytes.
// HBM-bound: 0.5 + 1/64 bytes in and 2 bytes out per weight, plus A and B
// (read from L2 by every tile).
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kMgN = 64;            // rows per tile
constexpr int kMgK = 128;           // columns per tile
constexpr int kMgLdA = kMgK + 16;   // A chunk row stride (elements): transpose reads conflict-free
constexpr int kMgLdP = kMgK + 8;    // product row stride (floats)

__global__ void __launch_bounds__(256)
k_merge(const uint8_t* __restrict__ packed, const uint8_t* __restrict__ codes,
        const float* __restrict__ scales, const float* __restrict__ mean_p, int64_t N, int64_t K,
        const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r, float s,
        uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t as[16 * kMgLdA];
  __shared__ __attribute__((aligned(16))) float prod[kMgN * kMgLdP];
  __shared__ float q4[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  if (tid < 16) q4[tid] = nf4_level(tid);
  const int64_t k0 = (int64_t)blockIdx.x * kMgK, n0 = (int64_t)blockIdx.y * kMgN;

  // The stored weight of this thread's four runs of 8 (step 3) is loaded
  // first, so that its latency overlaps the adapter product.  In round q
  // thread t takes row 16 q + t / 16 and columns 8 (t % 16) .. +7 of the
  // tile (runs outside the weight load nothing and are not stored).
  const int64_t nkb = K / kBlock;
  uint32_t pword[4], pcode[4];
  float pscale[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rn = 16 * q + (tid >> 4), kc = 8 * (tid & 15);
    const int64_t n = n0 + rn, k = k0 + kc;
    pword[q] = 0u; pcode[q] = 0u; pscale[q] = 0.0f;
    if (n < N && k < K) {
      const int64_t blk = n * nkb + k / kBlock;
      pword[q] = *reinterpret_cast<const uint32_t*>(packed + (n * K + k) / 2);
      pcode[q] = codes[blk];
      pscale[q] = scales[blk / kDQBlock];
    }
  }

  // Transpose-read addresses for the B-operand (A^T chunk: 16 r x 32 k of
  // this wave): group of 16 lanes = columns 32 w + 16 (grp & 1) .. +15,
  // rows 8 (grp >> 1) + 4 half .. +3.
  const int grp = lane >> 4, t = lane & 15;
  int ard[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    ard[half] = (8 * (grp >> 1) + 4 * half + (t >> 2)) * kMgLdA + 32 * wave + 16 * (grp & 1) + 4 * (t & 3);

  f32x16_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;

  for (int r0 = 0; r0 < r; r0 += 16) {
    // A chunk [16 r][128 k] into LDS: thread -> row tid / 16, 8 columns.
    {
      const int row = tid >> 4, col = (tid & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r0 + row < r && k0 + col < K)
        v = *reinterpret_cast<const uint4*>(A + (int64_t)(r0 + row) * K + k0 + col);
      *reinterpret_cast<uint4*>(as + row * kMgLdA + col) = v;
    }
    __syncthreads();
    const v4s_t lo = lds_read_tr16(as + ard[0]);
    const v4s_t hi = lds_read_tr16(as + ard[1]);
    typedef short v8s_t __attribute__((ext_vector_type(8)));
    const v8s_t bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bv);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t n = n0 + 32 * nb + c;
      uint4 av = make_uint4(0, 0, 0, 0);
      if (n < N && r0 + 8 * h < r) {
        const uint16_t* bp = B + n * r + r0 + 8 * h;
        if ((r & 7) == 0) {
          av = *reinterpret_cast<const uint4*>(bp);
        } else {   // rows of B are not 16-byte aligned: eight 2-byte loads, zero past r
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = r0 + 8 * h + i < r ? bp[i] : 0u;
          av = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                          e[6] | (e[7] << 16));
        }
      }
      acc[nb] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, av), bop, acc[nb]);
    }
    __syncthreads();   // before the next chunk overwrites `as`
  }

  // Accumulator nb: lane holds column 32 w + c and rows
  // 32 nb + 8 (v / 4) + 4 h + v % 4 of the tile.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      prod[(32 * nb + 8 * (v >> 2) + 4 * h + (v & 3)) * kMgLdP + 32 * wave + c] = acc[nb][v];
  __syncthreads();

  // Eight weights per thread and round (the runs loaded above), so each
  // store instruction of a wave writes four whole 256-byte row segments.
  const float mu = mean_p[0];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rn = 16 * q + (tid >> 4), kc = 8 * (tid & 15);
    const int64_t n = n0 + rn, k = k0 + kc;
    if (n >= N || k >= K) continue;
    float ah;
    {
#pragma clang fp contract(off)
      const float p = dq_level((int)pcode[q]) * pscale[q];
      ah = p + mu;
    }
    const uint32_t word = pword[q];
    const float* prow = prod + rn * kMgLdP + kc;
    const float4 p0 = *reinterpret_cast<const float4*>(prow);
    const float4 p1 = *reinterpret_cast<const float4*>(prow + 4);
    const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t byte = (word >> (8 * e)) & 0xffu;   // element 2e high, 2e+1 low nibble
      float wv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nib = j == 0 ? (int)(byte >> 4) : (int)(byte & 15u);
        float w;
        {
#pragma clang fp contract(off)
          w = q4[nib] * ah;
        }
        const float wh = bf16_to_f32(f32_to_bf16(w));     // the bf16 dequantised weight
        wv[j] = __builtin_fmaf(s, pv[2 * e + j], wh);
      }
      o[e] = pack_bf16x2(wv[0], wv[1]);
    }
    *reinterpret_cast<uint4*>(out + n * K + k) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_merge(const NF4Weight& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        uint16_t* out, hipStream_t st) {
  const dim3 grid((unsigned)((w.K + kMgK - 1) / kMgK), (unsigned)((w.N + kMgN - 1) / kMgN));
  hipLaunchKernelGGL(k_merge, grid, dim3(256), 0, st, w.packed, w.codes, w.scales, w.mean, w.N, w.K,
                     A, B, r, s, out);
  return hipGetLastError();
}

}  // namespace qlk
