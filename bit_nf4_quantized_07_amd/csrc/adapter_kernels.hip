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

// ---------------------------------------------------------------------------
// The adapters' gradients for more than 16 tokens, both in one launch that
// reads each operand once and writes the results directly:
//
//   dA = s U^T X   ([r, K]),   dB = s dY^T T   ([N, r])
//                  (llm-compass "QLoRA", 方法与公式, the derivatives of the
//                   equation with respect to A and B; U = dY B)
//
// Both contract over the M tokens: O[c][j] = sum_m P[m][c] Q[m][j], with
// (P, Q) = (X, U) for dA (O = dA^T) and (dY, T) for dB (O = dB).  A
// workgroup owns 32 columns c of P and all r outputs and contracts over every
// token itself, so no partial sums go through memory and no second launch
// adds them:
//  * its four waves take every fourth 32-token chunk; lane L loads rows
//    L / 4 and 16 + L / 4 of a chunk's 32 x 32 piece of P (16 bytes each, the
//    four lanes of a row its 64 contiguous bytes) and 16 bytes of the chunk's
//    32 x r piece of Q per 16 columns of r;
//  * the pieces go through a per-wave LDS slab (row-major) and come back as
//    MFMA operands with the transposing LDS read: lane (i, g) of
//    v_mfma_f32_16x16x32_bf16 gets column i of rows 8 g .. 8 g + 7 of the
//    chunk, the same token order for both operands;
//  * a wave issues the loads of KB chunks together, and those of its next KB
//    chunks before it multiplies the first ones (two register sets), so two
//    batches are in flight per wave;
//  * the four waves' sums are added through LDS in the order 0, 1, 2, 3, then
//    scaled by s (one fp32 rounding each), so the result is reproducible;
//  * slice numbers are dealt so that the workgroups one XCD receives take
//    consecutive slices: the two 64-byte halves of a 128-byte line of P are
//    read by workgroups on the same XCD.
// Tokens past M and columns past the operand are loaded as zeros (r and the
// column counts are multiples of 8, so a 16-byte piece lies wholly inside or
// wholly outside).
constexpr int kGradCols = 32;     // columns of P per workgroup
constexpr int kGradChunk = 32;    // tokens per MFMA step
constexpr int kGradWaves = 4;

struct GradJob {
  const uint16_t* P;   // [M, ld] bf16
  int64_t ld;          // row length of P (elements)
  int64_t cols;        // columns of P contracted (a multiple of 8)
  const uint16_t* Q;   // [M, r] bf16
  float* out;          // trans: [r, cols] (dA); else [cols, r] (dB)
  int trans;
  int slices;          // workgroups of this job: ceil(cols / 32)
};

template <int RT, int KB>
__global__ void __launch_bounds__(kGradWaves * 64)
k_adapter_grads(GradJob ja, GradJob jb, int M, int r, float s) {
  constexpr int PE = kGradChunk * kGradCols;     // elements of a chunk's P piece
  constexpr int QW = 16 * RT;                    // row length of the Q piece
  constexpr int CE = PE + kGradChunk * QW;       // elements of a chunk in the slab
  __shared__ __attribute__((aligned(16))) uint16_t slab[kGradWaves][KB * CE];
  __shared__ __attribute__((aligned(16))) float red[kGradWaves - 1][2 * RT][64][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const bool first = (int)blockIdx.x < ja.slices;
  const uint16_t* const P = first ? ja.P : jb.P;
  const uint16_t* const Q = first ? ja.Q : jb.Q;
  float* const out = first ? ja.out : jb.out;
  const int64_t ld = first ? ja.ld : jb.ld, cols = first ? ja.cols : jb.cols;
  const int trans = first ? ja.trans : jb.trans;
  const int nsl = first ? ja.slices : jb.slices;
  const int lb = first ? (int)blockIdx.x : (int)blockIdx.x - ja.slices;
  const int full = (nsl / kXCDs) * kXCDs;
  const int sl = lb < full ? (lb % kXCDs) * (full / kXCDs) + lb / kXCDs : lb;
  const int64_t c0 = (int64_t)sl * kGradCols;

  const __amdgpu_buffer_rsrc_t rp = rsrc_whole(P, (uint32_t)((int64_t)M * ld * 2));
  const __amdgpu_buffer_rsrc_t rq = rsrc_whole(Q, (uint32_t)((int64_t)M * r * 2));
  // this lane's pieces within a chunk
  const int prow = lane >> 2;                    // + 16 h
  const int64_t pcol = c0 + 8 * (lane & 3);
  const bool pcol_ok = pcol < cols;
  uint16_t* const my = slab[wave];

  const int nchunks = (M + kGradChunk - 1) / kGradChunk;
  const int per_wave = (nchunks + kGradWaves - 1) / kGradWaves;
  const int nb = (per_wave + KB - 1) / KB;      // batches, the same for every wave

  f32x4_t acc[2][RT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[h][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto load = [&](int b, uint4 (&pv)[KB][2], uint4 (&qv)[KB][RT]) {
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const int m0 = ((b * KB + q) * kGradWaves + wave) * kGradChunk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = m0 + 16 * h + prow;
        const bool ok = m < M && pcol_ok;
        pv[q][h] = bload128s(rp, ok ? (uint32_t)(((int64_t)m * ld + pcol) * 2) : kOOB, 0);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int p = 64 * t + lane;             // piece p: row p / (2 RT), columns 8 (p % (2 RT))
        const int m = m0 + p / (2 * RT);
        const int j = 8 * (p % (2 * RT));
        const bool ok = m < M && j < r;
        qv[q][t] = bload128s(rq, ok ? (uint32_t)(((int64_t)m * r + j) * 2) : kOOB, 0);
      }
    }
  };
  auto consume = [&](const uint4 (&pv)[KB][2], const uint4 (&qv)[KB][RT]) {
    // A wave's LDS operations run in issue order: these stores land after the
    // previous batch's reads and before this batch's reads.
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      uint16_t* const c = my + q * CE;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<uint4*>(c + (16 * h + prow) * kGradCols + 8 * (lane & 3)) = pv[q][h];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int p = 64 * t + lane;
        *reinterpret_cast<uint4*>(c + PE + (p / (2 * RT)) * QW + 8 * (p % (2 * RT))) = qv[q][t];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    typedef short v8s_t __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const uint16_t* const c = my + q * CE;
      // source lane 4 s + u of a 16-lane group points at row 8 g + 4 e + s,
      // column 4 u of a 16-column band: lane i receives column i of the
      // band's four rows
      const int rr = 8 * g + (i >> 2), cc = 4 * (i & 3);
      bf16x8_t aop[2], bop[RT];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4s_t lo = lds_read_tr16(c + rr * kGradCols + 16 * h + cc);
        const v4s_t hi = lds_read_tr16(c + (rr + 4) * kGradCols + 16 * h + cc);
        const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        aop[h] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const v4s_t lo = lds_read_tr16(c + PE + rr * QW + 16 * t + cc);
        const v4s_t hi = lds_read_tr16(c + PE + (rr + 4) * QW + 16 * t + cc);
        const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bop[t] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[h][t] = mfma_16x16x32(aop[h], bop[t], acc[h][t]);
    }
  };

  uint4 pa[KB][2], qa[KB][RT], pb[KB][2], qb[KB][RT];
  load(0, pa, qa);
  for (int b = 0; b < nb; b += 2) {
    if (b + 1 < nb) load(b + 1, pb, qb);
    consume(pa, qa);
    if (b + 2 < nb) load(b + 2, pa, qa);
    if (b + 1 < nb) consume(pb, qb);
  }

  // acc[h][t][v] = O[c0 + 16 h + 4 g + v][16 t + i]
  if (wave > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < RT; ++t)
        *reinterpret_cast<f32x4_t*>(&red[wave - 1][h * RT + t][lane][0]) = acc[h][t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f32x4_t v = acc[h][t];
#pragma unroll
      for (int w = 0; w < kGradWaves - 1; ++w) {
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(&red[w][h * RT + t][lane][0]);
        v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
      }
      const int64_t c = c0 + 16 * h + 4 * g;     // c .. c + 3 (cols is a multiple of 8)
      const int j = 16 * t + i;
      if (c >= cols || j >= r) continue;
      if (trans) {
        *reinterpret_cast<f32x4_t*>(out + (int64_t)j * cols + c) =
            f32x4_t{s * v[0], s * v[1], s * v[2], s * v[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[(c + e) * r + j] = s * v[e];
      }
    }
}

bool adapter_grads_supported(int64_t M, int64_t K, int64_t N, int r) {
  return r >= 1 && r <= 64 && r % 8 == 0 && K % 8 == 0 && N % 8 == 0 &&
         M * K * 2 < ((int64_t)1 << 31) && M * N * 2 < ((int64_t)1 << 31) &&
         M * r * 2 < ((int64_t)1 << 31);
}

hipError_t launch_adapter_grads(const uint16_t* U, const uint16_t* X, const uint16_t* dY,
                                const uint16_t* T, int64_t M, int64_t K, int64_t N, int r,
                                float s, float* dA, float* dB, hipStream_t st) {
  if (!adapter_grads_supported(M, K, N, r)) return hipErrorInvalidValue;
  GradJob ja{X, K, K, U, dA, 1, (int)((K + kGradCols - 1) / kGradCols)};
  GradJob jb{dY, N, N, T, dB, 0, (int)((N + kGradCols - 1) / kGradCols)};
  const dim3 grid((unsigned)(ja.slices + jb.slices));
  const int tiles = (r + 15) / 16;
  if (tiles <= 1)
    hipLaunchKernelGGL((k_adapter_grads<1, 8>), grid, dim3(kGradWaves * 64), 0, st, ja, jb, (int)M, r, s);
  else if (tiles <= 2)
    hipLaunchKernelGGL((k_adapter_grads<2, 4>), grid, dim3(kGradWaves * 64), 0, st, ja, jb, (int)M, r, s);
  else
    hipLaunchKernelGGL((k_adapter_grads<4, 4>), grid, dim3(kGradWaves * 64), 0, st, ja, jb, (int)M, r, s);
  return hipGetLastError();
}

hipError_t launch_rank16(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W, bool transposed,
                         int r, uint16_t* out, hipStream_t st) {
  return transposed ? rank16_dispatch<true>(S, M, C, W, r, out, st)
                    : rank16_dispatch<false>(S, M, C, W, r, out, st);
}

}  // namespace qlk
