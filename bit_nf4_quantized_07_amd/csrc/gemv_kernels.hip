// Small-M forward of the QLoRA linear layer (M <= 16 tokens): the layer is
// bound by streaming the packed NF4 weight from HBM once.
//
//   Y = X W_hat^T + s T B^T,   T = X A^T        (llm-compass "QLoRA",
//                                               方法与公式, the equation)
//
// Two kernels:
//  1. k_lora_down_partial: T = X A^T split over K into kTSplits partial sums
//     (fp32, workspace), one workgroup per (32 adapter rows, K slice).
//  2. k_gemv_nf4: workgroup = 4 waves = 64 weight rows (two groups of 32).
//     The four waves split K into quarters and reduce their partial products
//     through LDS in a fixed order.  Per 64-weight block, each lane loads the
//     16 contiguous packed bytes (32 nibbles) of one row that its lane group
//     covers, and v_mfma_f32_32x32x16_bf16 multiplies the zero-padded
//     activations with the UNSCALED bf16 NF4 levels of that block; the block's
//     a_hat is applied to the 32x32 partial product (a_hat is constant along
//     the block), so no weight is scaled element by element.  Loads run
//     kGemvDepth blocks ahead of the math; the 8-bit codes and second-level
//     scales are fetched 16 blocks at a time.  The prologue sums the T
//     partials in a fixed order into LDS; workgroup 0 also writes T (bf16) for
//     the backward.
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kGemvDepth = 4;
constexpr int kCodeRun = 16;     // codes fetched per 16-byte load

struct GemvStage {
  uint4 p[2];        // packed nibbles: rows of group 0 and 1, 32 per lane
  uint4 x[4];        // activations for the four MFMA steps of the block
};

template <int MAXM>
__global__ void __launch_bounds__(256)
k_gemv_nf4(const uint16_t* __restrict__ X, int M, NF4Weight w, const float* __restrict__ Tpart,
           const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y,
           uint16_t* __restrict__ T_out) {
  __shared__ uint32_t lut[256];   // byte -> (level of high nibble, level of low nibble), bf16
  __shared__ float q8[256];
  __shared__ float red[4][2][16][64];
  __shared__ float tl[kGemvMaxM * 256];
  const int tid = threadIdx.x;
  lut[tid] = pack_bf16x2(nf4_level(tid >> 4), nf4_level(tid & 15));
  q8[tid] = dq_level(tid);
  // T = sum of the split partials, fixed order
  for (int i = tid; i < M * r; i += 256) {
    float t = 0.0f;
    for (int z = 0; z < kTSplits; ++z) t += Tpart[(int64_t)z * M * r + i];
    tl[i] = t;
    if (blockIdx.x == 0) T_out[i] = f32_to_bf16(t);
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int64_t N = w.N, K = w.K, nkb = K / kBlock;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  int64_t nrow[2];
  bool nvalid[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    nrow[g] = n0 + 32 * g + c;
    nvalid[g] = nrow[g] < N;
  }
  const bool mvalid = c < M;
  const float mean = w.mean[0];
  const int64_t kb0 = wave * nkb / 4, kb1 = (wave + 1) * nkb / 4;
  const uint16_t* xrow = X + (int64_t)(mvalid ? c : 0) * K + 32 * h;
  // 16-byte code loads need 16-aligned runs (K a multiple of 4096); else bytes
  const bool bulk = (nkb % (4 * kCodeRun)) == 0;

  auto load = [&](GemvStage& st, int64_t kb) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      st.p[g] = make_uint4(0, 0, 0, 0);
      if (nvalid[g])
        st.p[g] = *reinterpret_cast<const uint4*>(w.packed + nrow[g] * (K / 2) + kb * 32 + 16 * h);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st.x[t] = make_uint4(0, 0, 0, 0);
      if (mvalid) st.x[t] = *reinterpret_cast<const uint4*>(xrow + kb * 64 + 8 * t);
    }
  };

  // Codes and scales of the current run of kCodeRun blocks (and the next run,
  // fetched one run ahead).  A run never straddles a 256-constant scale group
  // because runs start at multiples of 16 constants.
  uint4 crun[2], cnext[2];
  float srun[2], snext[2];
  auto load_run = [&](uint4 (&cr)[2], float (&sr)[2], int64_t kb) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      cr[g] = make_uint4(0, 0, 0, 0);
      sr[g] = 0.0f;
      if (nvalid[g]) {
        const int64_t b0 = nrow[g] * nkb + kb;
        cr[g] = *reinterpret_cast<const uint4*>(w.codes + b0);
        sr[g] = w.scales[b0 / kDQBlock];
      }
    }
  };
  auto code_of = [&](int g, int64_t kb) -> uint32_t {
    if (!bulk) return nvalid[g] ? w.codes[nrow[g] * nkb + kb] : 0u;
    // the run is rotated by one word every 4 blocks, so the current block's
    // code is always in word x (no dynamically indexed register array)
    return (crun[g].x >> (8 * (int)(kb & 3))) & 0xffu;
  };
  auto scale_of = [&](int g, int64_t kb) -> float {
    if (bulk) return srun[g];
    return nvalid[g] ? w.scales[(nrow[g] * nkb + kb) / kDQBlock] : 0.0f;
  };
  if (bulk) {
    load_run(crun, srun, kb0);
    if (kb0 + kCodeRun < kb1) load_run(cnext, snext, kb0 + kCodeRun);
  }

  f32x16_t acc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[g][v] = 0.0f;

  auto compute = [&](const GemvStage& st, int64_t kb) {
    if (bulk && kb != kb0 && kb % kCodeRun == 0) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        crun[g] = cnext[g];
        srun[g] = snext[g];
      }
      if (kb + kCodeRun < kb1) load_run(cnext, snext, kb + kCodeRun);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float ah = nvalid[g] ? absmax_decode_tab((int)code_of(g, kb), scale_of(g, kb), mean, q8) : 0.0f;
      const uint32_t pw[4] = {st.p[g].x, st.p[g].y, st.p[g].z, st.p[g].w};
      f32x16_t part;
#pragma unroll
      for (int v = 0; v < 16; ++v) part[v] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // word t holds the nibbles of k = 32h + 8t .. +7 (element 2b in the
        // high nibble of byte b); the lut gives both levels of a byte at once
        uint32_t o[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = lut[(pw[t] >> (8 * b)) & 0xffu];
        const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
        part = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, st.x[t]), bw, part);
      }
      // accumulator rows (tokens) 8*(v/4) + 4*h + v%4; only rows < MAXM matter
#pragma unroll
      for (int v = 0; v < (MAXM > 16 ? 16 : 8); ++v) acc[g][v] += ah * part[v];
    }
    if (bulk && (kb & 3) == 3) {
#pragma unroll
      for (int g = 0; g < 2; ++g) crun[g] = make_uint4(crun[g].y, crun[g].z, crun[g].w, 0u);
    }
  };

  GemvStage st[kGemvDepth];
#pragma unroll
  for (int i = 0; i < kGemvDepth; ++i)
    if (kb0 + i < kb1) load(st[i], kb0 + i);
  for (int64_t kb = kb0; kb < kb1; kb += kGemvDepth) {
#pragma unroll
    for (int i = 0; i < kGemvDepth; ++i) {
      if (kb + i < kb1) {
        compute(st[i], kb + i);
        if (kb + i + kGemvDepth < kb1) load(st[i], kb + i + kGemvDepth);
      }
    }
  }

  // Reduce the four K-quarters in a fixed order, add the adapter term, store.
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave][g][v][lane] = acc[g][v];
  __syncthreads();
  const int g = wave & 1;
  const int vbeg = (wave >> 1) * 8;
  if (!nvalid[g]) return;
  const int64_t n = nrow[g];
  for (int v = vbeg; v < vbeg + 8; ++v) {
    const int m = (v >> 2) * 8 + 4 * h + (v & 3);
    if (m < M) {
      const float base = ((red[0][g][v][lane] + red[1][g][v][lane]) + red[2][g][v][lane]) +
                         red[3][g][v][lane];
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l += tl[m * r + j] * bf16_to_f32(B[n * r + j]);
      Y[(int64_t)m * N + n] = f32_to_bf16(base + s * l);
    }
  }
}

// Partial sums of T = X A^T for M <= 16 over kTSplits slices of K: workgroup
// (jt, z) covers adapter rows 32*jt .. +31 and K slice z; its four waves take
// a quarter of the slice each and are reduced through LDS in a fixed order.
// MFMA rows = tokens (zero-padded), columns = adapter rows.
__global__ void __launch_bounds__(256)
k_lora_down_partial(const uint16_t* __restrict__ X, int M, int64_t K, const uint16_t* __restrict__ A,
                    int r, float* __restrict__ Tpart) {
  __shared__ float red[4][8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int j = blockIdx.x * 32 + c;
  const int z = blockIdx.y;
  const bool jvalid = j < r, mvalid = c < M;
  const int64_t nkb = K / kBlock;
  const int64_t zb0 = z * nkb / kTSplits, zb1 = (z + 1) * nkb / kTSplits;
  const int64_t kb0 = zb0 + wave * (zb1 - zb0) / 4, kb1 = zb0 + (wave + 1) * (zb1 - zb0) / 4;
  const uint16_t* xrow = X + (int64_t)(mvalid ? c : 0) * K + 32 * h;
  const uint16_t* arow = A + (int64_t)(jvalid ? j : 0) * K + 32 * h;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    uint4 xa[4], aa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      xa[t] = mvalid ? *reinterpret_cast<const uint4*>(xrow + kb * 64 + 8 * t) : make_uint4(0, 0, 0, 0);
      aa[t] = jvalid ? *reinterpret_cast<const uint4*>(arow + kb * 64 + 8 * t) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, xa[t]), __builtin_bit_cast(bf16x8_t, aa[t]), acc);
  }
  // rows 8*(v/4) + 4*h + v%4 (tokens) of which only < 16 matter (v < 8)
#pragma unroll
  for (int v = 0; v < 8; ++v) red[wave][v][lane] = acc[v];
  __syncthreads();
  if (wave == 0) {
    for (int v = 0; v < 8; ++v) {
      const int m = (v >> 2) * 8 + 4 * h + (v & 3);
      if (m < M && jvalid) {
        const float sum = ((red[0][v][lane] + red[1][v][lane]) + red[2][v][lane]) + red[3][v][lane];
        Tpart[((int64_t)z * M + m) * r + j] = sum;
      }
    }
  }
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                       const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T, float* Tpart,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_lora_down_partial, dim3((r + 31) / 32, kTSplits), dim3(256), 0, st, X,
                     (int)M, w.K, A, r, Tpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((w.N + 63) / 64);
  timer_begin(TK_GEMV, st);
  hipLaunchKernelGGL(k_gemv_nf4<16>, dim3(grid), dim3(256), 0, st, X, (int)M, w, Tpart, B, r, s, Y, T);
  timer_end(TK_GEMV, st);
  return hipGetLastError();
}

}  // namespace qlk
