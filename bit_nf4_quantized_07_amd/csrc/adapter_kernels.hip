// Rank-r projections of the adapter for more than 16 tokens:
//
//   T = X A^T   (forward, and the backward when T was not saved)
//   U = dY B    (backward)             (llm-compass "QLoRA", 方法与公式, the
//                                       equation and its derivative)
//
// out[m][j] = sum_c S[m][c] W(j, c), with S = X or dY ([M, C], bf16) and
// W(j, c) = A[j][c] (contraction contiguous) or B[c][j] (transposed).
// One workgroup owns 16 rows of S (or 8, with the MFMA's other 8 rows zero,
// when 16-row tiles would leave CUs idle) and all r outputs; its NW waves take every
// NW-th 64-wide slice of the contraction (v_mfma_f32_16x16x32_bf16, S read
// once in total), and the NW partial sums are added through LDS in a fixed
// order, so the bf16 result is written by the same kernel and is
// bit-reproducible.  A wave issues the loads of several slices before their
// MFMAs (branch-free: out-of-range pieces are loaded from a valid address and
// replaced by zeros), so that many loads are in flight per wave.  W(j, c) =
// B[c][j] is loaded as rows of B (16 bytes per lane, coalesced) and
// transposed through a 1 KB slice of LDS per wave by the transposing LDS
// read; r and C are multiples of 8, so every 16-byte piece is wholly inside
// or wholly outside the operands.
#include <type_traits>

#include "dequant_block.h"
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kRankRows = 16;
constexpr int kRankMaxTiles = 16;   // r <= 256

// Contraction slices whose loads one wave issues together (registers:
// 8 (1 + RT) per slice).  In the launch shared with the dequantisation the
// batch is smaller, so that the kernel keeps to 64 VGPRs at r <= 16 and runs
// two 1024-thread workgroups per CU for the dequantising workgroups.
template <int RT>
constexpr int rank_batch() { return RT <= 1 ? 4 : (RT <= 2 ? 2 : 1); }
template <int RT>
constexpr int rank_batch_shared() { return RT <= 1 ? 2 : 1; }

// v if ok, else zeros (component-wise: a select of the struct would go
// through private memory).
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// One workgroup's share; `blk` is its index in the rank-r grid.
//
// A slice is 64 contraction indices, two MFMAs.  Lane (row, grp) loads the
// 16 contiguous indices 16 grp .. 16 grp + 15 of the slice (two 16-byte
// loads), so that the four lanes of a row cover its 128 bytes and every
// cache line fetched is used whole; MFMA h takes indices 16 grp + 8 h .. +7
// of every lane, the same permutation of the slice for both operands.
template <bool WT, int RT, int NW, int kB>
__device__ __forceinline__ void rank16_block(const uint16_t* __restrict__ S, int M, int64_t C,
                                             const uint16_t* __restrict__ W, int r, int rows,
                                             uint16_t* __restrict__ out, int blk) {
  __shared__ float red[NW - 1][kRankRows][RT * 16];
  // WT: one 64 (c) x 16 (j) slice of B per wave, row-major.
  __shared__ __attribute__((aligned(16))) uint16_t slab[WT ? NW : 1][64 * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int m0 = blk * rows;
  const int m = m0 + row;
  const bool mvalid = row < rows && m < M;
  const int64_t nsteps = (C + 63) / 64;
  const uint16_t* srow = S + (int64_t)(mvalid ? m : 0) * C;
  // WT: lane L loads rows c0 + L / 2 and c0 + 32 + L / 2 of the slice,
  // columns 8 (L % 2) .. +7, and reads back column `row` of rows
  // 16 grp + 8 h .. +7 for MFMA h (transposing reads of four rows each).
  const int wrow = lane >> 1, wcol = 8 * (lane & 1);
  uint16_t* const my = slab[WT ? wave : 0];
  const int rd = (16 * grp + (row >> 2)) * 16 + 4 * (row & 3);

  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t base = wave; base < nsteps; base += (int64_t)NW * kB) {
    uint4 xv[kB][2], wv[kB][RT][2];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int64_t ks = base + (int64_t)NW * b;
      const bool sv = ks < nsteps;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t k = ks * 64 + 16 * grp + 8 * h;   // 8 contraction indices
        const bool kvalid = sv && k < C;
        const uint4 v = *reinterpret_cast<const uint4*>(srow + (kvalid ? k : 0));
        xv[b][h] = keep_if(mvalid && kvalid, v);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          if (!WT) {
            const int j = 16 * t + row;
            const bool ok = kvalid && j < r;
            const uint4 w = *reinterpret_cast<const uint4*>(W + (ok ? (int64_t)j * C + k : 0));
            wv[b][t][h] = keep_if(ok, w);
          } else {
            const int64_t c = ks * 64 + 32 * h + wrow;
            const int j = 16 * t + wcol;
            const bool ok = sv && c < C && j < r;
            const uint4 w = *reinterpret_cast<const uint4*>(W + (ok ? c * r + j : 0));
            wv[b][t][h] = keep_if(ok, w);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch before the first MFMA
#pragma unroll
    for (int b = 0; b < kB; ++b) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        bf16x8_t bop[2];
        if (!WT) {
          bop[0] = __builtin_bit_cast(bf16x8_t, wv[b][t][0]);
          bop[1] = __builtin_bit_cast(bf16x8_t, wv[b][t][1]);
        } else {
          // A wave's LDS operations run in issue order: the stores are
          // complete before the reads, which complete before the next stores.
          *reinterpret_cast<uint4*>(my + wrow * 16 + wcol) = wv[b][t][0];
          *reinterpret_cast<uint4*>(my + (32 + wrow) * 16 + wcol) = wv[b][t][1];
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const v4s_t lo = lds_read_tr16(my + rd + 8 * h * 16);
            const v4s_t hi = lds_read_tr16(my + rd + (8 * h + 4) * 16);
            typedef short v8s_t __attribute__((ext_vector_type(8)));
            const v8s_t bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            bop[h] = __builtin_bit_cast(bf16x8_t, bv);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc[t] = mfma_16x16x32(__builtin_bit_cast(bf16x8_t, xv[b][h]), bop[h], acc[t]);
      }
    }
  }

  // acc[t][v]: row 4 grp + v, column 16 t + row of the tile.  Waves 1..NW-1
  // hand their sums to wave 0, which adds them in the order 0, 1, ..., NW-1.
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave - 1][4 * grp + v][16 * t + row] = acc[t][v];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 16 * t + row;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = m0 + 4 * grp + v;
      float sum = acc[t][v];
#pragma unroll
      for (int q = 0; q < NW - 1; ++q) sum += red[q][4 * grp + v][j];
      if (4 * grp + v < rows && mm < M && j < r) out[(int64_t)mm * r + j] = f32_to_bf16(sum);
    }
  }
}

template <bool WT, int RT, int NW>
__global__ void __launch_bounds__(NW * 64)
k_rank16(const uint16_t* __restrict__ S, int M, int64_t C, const uint16_t* __restrict__ W, int r,
         int rows, uint16_t* __restrict__ out) {
  rank16_block<WT, RT, NW, rank_batch<RT>()>(S, M, C, W, r, rows, out, blockIdx.x);
}

// The backward's U = dY B and its one-off dequantisation of the weight are
// independent and each too short to fill the device for long: one launch
// runs both, the first `rank_blocks` workgroups computing U and the rest
// dequantising (each workgroup does one or the other, so the barriers inside
// each body see all of its threads).
template <bool WT, int RT, int NW>
__global__ void __launch_bounds__(NW * 64)
k_rank16_and_dequant(const uint16_t* __restrict__ S, int M, int64_t C,
                     const uint16_t* __restrict__ W, int r, int rows, uint16_t* __restrict__ out,
                     int rank_blocks, const uint8_t* __restrict__ packed,
                     const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                     const float* __restrict__ mean, int64_t nwords, Codebook4 cb,
                     uint16_t* __restrict__ wout) {
  if ((int)blockIdx.x < rank_blocks)
    rank16_block<WT, RT, NW, rank_batch_shared<RT>()>(S, M, C, W, r, rows, out, blockIdx.x);
  else
    nf4_dequant_block(packed, codes, scales, mean, nwords, cb, wout,
                      (int64_t)blockIdx.x - rank_blocks);
}

template <bool WT>
static hipError_t rank16_dispatch(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W, int r,
                                  uint16_t* out, hipStream_t st) {
  // 8 rows per workgroup when 16 would give fewer workgroups than CUs
  const int rows = (M + kRankRows - 1) / kRankRows < 256 ? 8 : kRankRows;
  const dim3 grid((unsigned)((M + rows - 1) / rows));
  const int tiles = (r + 15) / 16;
  // More waves (loads in flight) for small r; the LDS of the final sum bounds NW * r.
  if (tiles <= 1) hipLaunchKernelGGL((k_rank16<WT, 1, 16>), grid, dim3(1024), 0, st, S, (int)M, C, W, r, rows, out);
  else if (tiles <= 2) hipLaunchKernelGGL((k_rank16<WT, 2, 16>), grid, dim3(1024), 0, st, S, (int)M, C, W, r, rows, out);
  else if (tiles <= 4) hipLaunchKernelGGL((k_rank16<WT, 4, 8>), grid, dim3(512), 0, st, S, (int)M, C, W, r, rows, out);
  else if (tiles <= 8) hipLaunchKernelGGL((k_rank16<WT, 8, 4>), grid, dim3(256), 0, st, S, (int)M, C, W, r, rows, out);
  else hipLaunchKernelGGL((k_rank16<WT, kRankMaxTiles, 4>), grid, dim3(256), 0, st, S, (int)M, C, W, r, rows, out);
  return hipGetLastError();
}

hipError_t launch_rank16_and_dequant(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W,
                                     bool transposed, int r, uint16_t* out, const NF4Weight& w,
                                     uint16_t* wout, hipStream_t st, Span sp) {
  const int rows = (M + kRankRows - 1) / kRankRows < 256 ? 8 : kRankRows;
  const int rank_blocks = (int)((M + rows - 1) / rows);
  const int64_t nwords = w.N * w.K / 8;
  const Codebook4 cb = nf4_codebook4();
  const int tiles = (r + 15) / 16;
  auto go = [&](auto rt, auto nw) {
    constexpr int RT = decltype(rt)::value, NW = decltype(nw)::value;
    const int64_t dq_blocks = (nwords + NW * kDqWaveWords - 1) / (NW * kDqWaveWords);
    const dim3 grid((unsigned)(rank_blocks + dq_blocks));
    if (transposed)
      hipExtLaunchKernelGGL((k_rank16_and_dequant<true, RT, NW>), grid, dim3(NW * 64), 0, st,
                            sp.start, sp.stop, 0, S, (int)M, C, W, r, rows, out, rank_blocks,
                            w.packed, w.codes, w.scales, w.mean, nwords, cb, wout);
    else
      hipExtLaunchKernelGGL((k_rank16_and_dequant<false, RT, NW>), grid, dim3(NW * 64), 0, st,
                            sp.start, sp.stop, 0, S, (int)M, C, W, r, rows, out, rank_blocks,
                            w.packed, w.codes, w.scales, w.mean, nwords, cb, wout);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  if (tiles <= 1) go(I1(), I16());
  else if (tiles <= 2) go(I2(), I16());
  else if (tiles <= 4) go(I4(), I8());
  else if (tiles <= 8) go(I8(), I4());
  else go(std::integral_constant<int, kRankMaxTiles>(), I4());
  return hipGetLastError();
}

hipError_t launch_rank16(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W, bool transposed,
                         int r, uint16_t* out, hipStream_t st) {
  return transposed ? rank16_dispatch<true>(S, M, C, W, r, out, st)
                    : rank16_dispatch<false>(S, M, C, W, r, out, st);
}

}  // namespace qlk
