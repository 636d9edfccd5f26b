// Small-M forward of the QLoRA linear layer (M <= 16 tokens): the layer is
// bound by streaming the packed NF4 weight from HBM once.
//
//   Y = X W_hat^T + s T B^T,   T = X A^T        (llm-compass "QLoRA",
//                                               方法与公式, the equation)
//
// Two kernels:
//  1. k_lora_down_partial: T = X A^T split over K into kTSplits partial sums
//     (fp32, workspace), one workgroup per (32 adapter rows, K slice).
//  2. the weight stream, which adds the partials in a fixed order: the split
//     kernel k_gemv_split further below where its shapes allow, else
//     k_gemv_dma / k_gemv_nf4.
//     k_gemv_nf4: workgroup = 4 waves = 64 weight rows (two groups of 32).
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
#include <type_traits>

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

// Streaming variant of the small-M forward (taken when K / 64 is a multiple
// of 16).  Same workgroup shape and arithmetic as k_gemv_nf4, but the packed
// weight goes through LDS: per super-step of 4 blocks, a wave fetches its 64
// rows x 128 bytes with 8 buffer loads that write LDS directly (8 rows x 128
// contiguous bytes per load instead of 32 rows x 32 bytes), one super-step
// ahead into the other of two LDS stages, and reads the MFMA operands back
// from LDS.  The 16-byte pieces of
// row i are XOR-swizzled by (i >> 1) & 7 so that the operand reads are
// conflict-free.  Each wave owns its LDS region, so no barrier is needed in
// the loop.  The activations of a super-step are loaded one super-step ahead
// into registers; the 8-bit codes (4 per row) and the scale come with them.
constexpr int kGemvSS = 4;                      // blocks per super-step
constexpr int kGemvStage = 64 * 128;            // bytes per wave and stage
// s_waitcnt immediate (gfx9 encoding): vmcnt <= 28, expcnt and lgkmcnt not waited on.
constexpr int kGemvWaitVm28 = (28 & 0xF) | ((28 >> 4) << 14) | (0x7 << 4) | (0xF << 8);

struct GemvSSRegs {
  uint4 x[kGemvSS][4];    // activations: block b, MFMA step t
  uint32_t code[2];       // 4 codes of row group g (byte b = block b)
  float sc[2];
};

template <int MAXM>
__global__ void __launch_bounds__(256)
k_gemv_dma(const uint16_t* __restrict__ X, int M, NF4Weight w, const float* __restrict__ Tpart,
           const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y,
           uint16_t* __restrict__ T_out) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[4 * kGemvStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[4 * kGemvStage];
  __shared__ uint32_t lut[256];   // byte -> (level of high nibble, level of low nibble), bf16
  __shared__ float q8[256];
  __shared__ uint16_t tl[kGemvMaxM * 256];   // T, bf16
  const int tid = threadIdx.x;
  lut[tid] = pack_bf16x2(nf4_level(tid >> 4), nf4_level(tid & 15));
  q8[tid] = dq_level(tid);
  for (int i = tid; i < M * r; i += 256) {
    float t = 0.0f;
    for (int z = 0; z < kTSplits; ++z) t += Tpart[(int64_t)z * M * r + i];
    tl[i] = f32_to_bf16(t);
    if (blockIdx.x == 0) T_out[i] = tl[i];
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int64_t q = nkb / 4;                 // blocks per wave (a multiple of 4)
  const int64_t kb0 = wave * q;
  const int nss = (int)(q / kGemvSS);
  uint8_t* const my0 = st0 + wave * kGemvStage;
  uint8_t* const my1 = st1 + wave * kGemvStage;

  // Weight loads: load i fills rows 8i .. 8i+7 of the wave's 64; lane L lands
  // at 16 L: row 8i + L/8, physical piece L%8 = logical piece (L%8) ^ swz.
  auto swz = [](int row) { return (row >> 1) & 7; };
  const uint32_t pbytes = (uint32_t)(N * (K / 2));
  uint32_t poff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int piece = (lane & 7) ^ swz(row);
    poff[i] = n0 + row < N ? (uint32_t)((n0 + row) * (K / 2) + piece * 16) : kOOB;
  }
  const __amdgpu_buffer_rsrc_t rp = rsrc_whole(w.packed, pbytes);
  auto load_w = [&](uint8_t* buf, int ss) {
    const uint32_t soff = (uint32_t)(kb0 + (int64_t)__builtin_amdgcn_readfirstlane(ss) * kGemvSS) * 32u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rp, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, poff[i], soff, 0, 0);
  };
  // Operand of block b, half h, group g: row 32 g + c, logical piece 2 b + h.
  auto wfrag = [&](const uint8_t* buf, int g, int b) -> uint4 {
    const int row = 32 * g + c;
    return *reinterpret_cast<const uint4*>(buf + row * 128 + (((2 * b + h) ^ swz(row)) * 16));
  };
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const uint32_t xoff = mvalid ? (uint32_t)(((int64_t)c * K + 32 * h) * 2) : kOOB;
  const uint32_t cbytes = (uint32_t)(N * nkb);
  const uint32_t sbytes = (uint32_t)(((N * nkb + kDQBlock - 1) / kDQBlock) * 4);
  const __amdgpu_buffer_rsrc_t rx = rsrc_whole(X, xbytes);
  const __amdgpu_buffer_rsrc_t rc = rsrc_whole(w.codes, cbytes);
  const __amdgpu_buffer_rsrc_t rsc = rsrc_whole(w.scales, sbytes);
  uint32_t coff[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) coff[g] = nvalid[g] ? (uint32_t)(nrow[g] * nkb + kb0) : kOOB;
  auto load_r = [&](GemvSSRegs& R, int ss) {
    const uint32_t kbs = (uint32_t)__builtin_amdgcn_readfirstlane(ss) * kGemvSS;   // from kb0
    const uint32_t xs = (uint32_t)(kb0 + kbs) * (kBlock * 2);
#pragma unroll
    for (int b = 0; b < kGemvSS; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        R.x[b][t] = bload128s(rx, xoff == kOOB ? kOOB : xoff + (uint32_t)(b * 128 + t * 16), xs);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      R.code[g] = bload32s(rc, coff[g], kbs);
      R.sc[g] = __uint_as_float(
          bload32(rsc, coff[g] == kOOB ? kOOB : ((coff[g] + kbs) / kDQBlock) * 4u));
    }
  };

  f32x16_t acc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[g][v] = 0.0f;

  auto compute = [&](const uint8_t* buf, const GemvSSRegs& R) {
#pragma unroll
    for (int b = 0; b < kGemvSS; ++b)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float ah = absmax_decode_tab((int)((R.code[g] >> (8 * b)) & 0xffu), R.sc[g], mean, q8);
        const uint4 pv = wfrag(buf, g, b);
        const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w};
        f32x16_t part;
#pragma unroll
        for (int v = 0; v < 16; ++v) part[v] = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = lut[(pw[t] >> (8 * e)) & 0xffu];
          part = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, R.x[b][t]),
                               __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3])), part);
        }
#pragma unroll
        for (int v = 0; v < (MAXM > 16 ? 16 : 8); ++v) acc[g][v] += ah * part[v];
      }
  };

  // Super-step ss uses LDS stage ss % 2 and register set ss % 2.  At its
  // start the loads of ss+1 are issued (8 weight, 16 activation, 4 code and
  // scale loads), after which waiting for at most 28 outstanding loads means
  // that everything of ss has arrived.
  GemvSSRegs rg[2];
  load_w(my0, 0);
  load_r(rg[0], 0);
  auto sstep = [&](auto Pc, int ss) {
    constexpr int P = decltype(Pc)::value;
    uint8_t* cur = P == 0 ? my0 : my1;
    uint8_t* nxt = P == 0 ? my1 : my0;
    if (ss + 1 < nss) {
      load_w(nxt, ss + 1);
      load_r(rg[(P + 1) % 2], ss + 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kGemvWaitVm28);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, rg[P]);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int ss = 0; ss < nss; ss += 2) {
    sstep(std::integral_constant<int, 0>(), ss);
    if (ss + 1 < nss) sstep(std::integral_constant<int, 1>(), ss + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Reduce the four K-quarters in a fixed order (through this wave's own
  // stage-0 region), add the adapter term, store.
  float* red = reinterpret_cast<float*>(st0);   // [wave][g][v][lane]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((wave * 2 + g) * 16 + v) * 64 + lane] = acc[g][v];
  __syncthreads();
  const int g = wave & 1;
  const int vbeg = (wave >> 1) * 8;
  if (!nvalid[g]) return;
  const int64_t n = nrow[g];
  for (int v = vbeg; v < vbeg + 8; ++v) {
    const int m = (v >> 2) * 8 + 4 * h + (v & 3);
    if (m < M) {
      float base = red[((0 * 2 + g) * 16 + v) * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) base += red[((ww * 2 + g) * 16 + v) * 64 + lane];
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l += bf16_to_f32(tl[m * r + j]) * bf16_to_f32(B[n * r + j]);
      Y[(int64_t)m * N + n] = f32_to_bf16(base + s * l);
    }
  }
}

// Partial sums of T = X A^T for M <= 16 over kTSplits slices of K: workgroup
// (jt, z) covers adapter rows 32*jt .. +31 and K slice z; its eight waves
// take an eighth of the slice each (one 64-block on K = 8192, so every load
// of the kernel is in flight at once) and are reduced through LDS in a fixed
// order.  MFMA rows = tokens (zero-padded), columns = adapter rows.
constexpr int kTWaves = 8;

__global__ void __launch_bounds__(64 * kTWaves)
k_lora_down_partial(const uint16_t* __restrict__ X, int M, int64_t K, const uint16_t* __restrict__ A,
                    int r, float* __restrict__ Tpart) {
  __shared__ float red[kTWaves][8][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int j = blockIdx.x * 32 + c;
  const int z = blockIdx.y;
  const bool jvalid = j < r, mvalid = c < M;
  const int64_t nkb = K / kBlock;
  const int64_t zb0 = z * nkb / kTSplits, zb1 = (z + 1) * nkb / kTSplits;
  const int64_t kb0 = zb0 + wave * (zb1 - zb0) / kTWaves, kb1 = zb0 + (wave + 1) * (zb1 - zb0) / kTWaves;
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
        float sum = red[0][v][lane];
        for (int ww = 1; ww < kTWaves; ++ww) sum += red[ww][v][lane];
        Tpart[((int64_t)z * M + m) * r + j] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M forward with the contraction split over the waves of a workgroup
// (k_gemv_split), taken when K is 2048, 4096 or 8192, r <= 64 and the weight
// has at most 256 x 8 groups of 16 rows.
//
// The weight is read once from HBM, so the kernel has to keep every CU
// streaming and spend as little issue time per weight as it can:
//  * one 512-thread workgroup per CU (at most 256 workgroups); each owns a run
//    of R rows (R a multiple of 16, the same for all but the last), so every
//    CU moves the same number of bytes;
//  * its 8 waves split K into 8 slices of S blocks; a wave keeps the
//    activations of its slice in registers (as MFMA operands) and walks the
//    workgroup's rows 16 at a time (a row group), so no activation is read
//    twice; each wave leaves its partial product of every row group in LDS
//    and the 8 slices are added once, at the end, in a fixed order (no
//    barrier in the loop);
//  * the weight goes straight from HBM into registers, 8 loads of 1 KB per
//    wave in flight (a ring that runs across row groups): for M <= 8, lane
//    (n = lane % 16, g = lane / 16) loads the 16 bytes [16 g, 16 g + 16) of
//    the 64-byte run of row n covering two blocks (groups 0-1 block b, groups
//    2-3 block b + 1); for M <= 16 the 8 bytes [8 g, 8 g + 8) of one block;
//  * each packed byte is decoded to its two bf16 NF4 levels by one LDS read
//    from a 64 KB table that gives every lane its own column (entry e of lane
//    L at byte e * 256 + 4 L), so the reads never conflict; the address is one
//    byte permute of the packed word and the lane's offset;
//  * v_mfma_f32_16x16x32_bf16 multiplies the unscaled levels (columns = weight
//    rows) with the zero-padded activations (rows = tokens); a_hat of the
//    block multiplies the 16 x 16 partial product afterwards.  For M <= 8 the
//    MFMA's 16 token rows hold the tokens of block b in rows 0-7 and those of
//    block b + 1 in rows 8-15 (each half's activations are zero in the other
//    block's lanes), so two blocks with different a_hat share one MFMA chain;
//  * T = Xa A^T comes from the 16 K-slice partials of k_lora_down_partial,
//    launched just before (16 small workgroups, one round trip of loads):
//    each workgroup adds them in a fixed order and rounds T once to bf16
//    before its weight stream starts, and workgroup 0 writes T.  Computing T
//    in every workgroup instead (all of A, 256 KB on K = 8192, through L2 in
//    eight dependent rounds per wave) held the weight stream back by 6 us;
//  * the adapter term s T B^T of each row group is one more MFMA chain over
//    r, and Y is rounded once.
//
//   Y = X W_hat^T + s T B^T,   T = Xa A^T   (llm-compass "QLoRA", 方法与公式,
//                                            the equation; Xa = X unless the
//                                            adapter input is dropped)
constexpr int kGsWaves = 8;
constexpr int kGsThreads = kGsWaves * 64;
constexpr int kGsMaxRG = 8;                      // row groups of 16 per workgroup
constexpr int kGsMaxRT = 4;                      // adapter tiles of 16 (r <= 64)
constexpr int kGsTable = 256 * 64;               // dwords: entry e, lane L at e * 64 + L
constexpr int kGsRing = 8;                       // weight loads in flight per wave

template <int S, bool PAIR>
struct GsShape {
  static constexpr int NU = PAIR ? S / 2 : S;    // load units per row group and wave
  static constexpr int MF = PAIR ? 4 : 2;        // MFMAs per unit
  static constexpr int CW = S / 4;               // code dwords per row and slice
  static constexpr int D = NU < kGsRing ? NU : kGsRing;
};

template <int S, bool PAIR, int MI, int RT>
__global__ void __launch_bounds__(kGsThreads)
k_gemv_split(const uint16_t* __restrict__ X, int M, NF4Weight w, const float* __restrict__ Tpart,
             const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y,
             uint16_t* __restrict__ T_out, int rows_wg) {
  using Sh = GsShape<S, PAIR>;
  constexpr int NU = Sh::NU, MF = Sh::MF, CW = Sh::CW, D = Sh::D;
  constexpr int PARTW = kGsWaves * 64 * MI;      // floats of one row group's partials
  __shared__ __attribute__((aligned(16))) uint32_t tbl[kGsTable];           // 64 KB
  __shared__ __attribute__((aligned(16))) float part[kGsMaxRG * PARTW];     // 16 or 64 KB
  __shared__ __attribute__((aligned(16))) uint16_t tl[kGemvMaxM * 16 * RT];   // T, bf16 [M][r]
  __shared__ float q8[256];                                                  // the 8-bit levels

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int64_t N = w.N, K = w.K, Kb = K / kBlock;
  const int64_t row0 = (int64_t)blockIdx.x * rows_wg;
  const int rgs = (int)((min((int64_t)rows_wg, N - row0) + 15) / 16);
  const int kb0 = wave * S;                        // first block of this wave's slice

  const __amdgpu_buffer_rsrc_t rw = rsrc_whole(w.packed, (uint32_t)(N * (K / 2)));
  const __amdgpu_buffer_rsrc_t rc = rsrc_whole(w.codes, (uint32_t)(N * Kb));
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_whole(w.scales, (uint32_t)(((N * Kb + kDQBlock - 1) / kDQBlock) * 4));

  // --- the weight ring: unit u of row group jr goes to slot u % D ---------
  uint4 wu[D];
  uint32_t cw[CW];
  float sc;
  auto row_of = [&](int jr) -> int64_t { return row0 + 16 * jr + col; };
  auto load_unit = [&](int jr, int u) {
    const int64_t n = row_of(jr);
    if (PAIR) {
      const uint32_t off = n < N ? (uint32_t)(n * (K / 2) + (kb0 + 2 * u) * 32 + 16 * g) : kOOB;
      wu[u % D] = bload128s(rw, off, 0);
    } else {
      const uint32_t off = n < N ? (uint32_t)(n * (K / 2) + (kb0 + u) * 32 + 8 * g) : kOOB;
      const uint2 v = bload64s(rw, off, 0);
      wu[u % D] = make_uint4(v.x, v.y, 0u, 0u);
    }
  };
  auto load_consts = [&](int jr) {   // the slice's 8-bit codes of row n and its scale
    const int64_t n = row_of(jr);
    const bool ok = n < N;
    const uint32_t coff = ok ? (uint32_t)(n * Kb + kb0) : kOOB;
    if constexpr (CW == 4) {
      const uint4 v = bload128s(rc, coff, 0);
      cw[0] = v.x; cw[1] = v.y; cw[2] = v.z; cw[3] = v.w;
    } else if constexpr (CW == 2) {
      const uint2 v = bload64s(rc, coff, 0);
      cw[0] = v.x; cw[1] = v.y;
    } else {
      cw[0] = bload32s(rc, coff, 0);
    }
    sc = __uint_as_float(bload32s(rs, ok ? (uint32_t)((n * Kb + kb0) / kDQBlock) * 4u : kOOB, 0));
  };
  // The first loads go out before anything else, so that they are in flight
  // while the table, the activations and T are prepared.
#pragma unroll
  for (int u = 0; u < D; ++u) load_unit(0, u);
  load_consts(0);
  const float mean = w.mean[0];

  // B rows of row group `wave`, for its adapter term at the end: one 16-byte
  // piece per lane and 32 of r (r is a multiple of 8).
  constexpr int BCH = (RT + 1) / 2;
  const int64_t bn = row0 + 16 * wave + col;
  const bool bvalid = wave < rgs && bn < N;
  const __amdgpu_buffer_rsrc_t rb = rsrc_whole(B, (uint32_t)(N * r * 2));
  uint4 bpre[BCH];
#pragma unroll
  for (int c = 0; c < BCH; ++c)
    bpre[c] = bload128s(rb, bvalid && 32 * c + 8 * g < r ? (uint32_t)((bn * r + 32 * c + 8 * g) * 2) : kOOB, 0);

  if (tid < 256) q8[tid] = dq_level(tid);
  // --- the byte -> (level of the high nibble, level of the low nibble)
  // table, one column per lane.  Thread t fills entries e = 8 k + t / 64 of
  // its lane's column.
#pragma unroll
  for (int k = 0; k < 256 / kGsWaves; ++k) {
    const int e = kGsWaves * k + (tid >> 6);
    tbl[k * kGsThreads + tid] = pack_bf16x2(nf4_level(e >> 4), nf4_level(e & 15));
  }
  const uint32_t lane4 = (uint32_t)lane * 4u;

  // --- activations of the slice as MFMA operands (rows = tokens) -----------
  bf16x8_t xop[NU][MF];
  auto load_x = [&](const uint16_t* src) {
    const __amdgpu_buffer_rsrc_t rx = rsrc_whole(src, (uint32_t)((int64_t)M * K * 2));
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        int t, blk, k;
        bool ok;
        if (PAIR) {
          const int half = col >> 3;
          t = col & 7;
          blk = kb0 + 2 * u + half;
          k = 32 * (g & 1) + 8 * j;
          ok = half == (g >> 1) && t < M;
        } else {
          t = col;
          blk = kb0 + u;
          k = 16 * g + 8 * j;
          ok = t < M;
        }
        const uint32_t off = ok ? (uint32_t)(((int64_t)t * K + (int64_t)blk * kBlock + k) * 2) : kOOB;
        xop[u][j] = __builtin_bit_cast(bf16x8_t, bload128s(rx, off, 0));
      }
  };
  load_x(X);

  // --- T = the sum of the partials (fixed order), rounded once to bf16 ------
  for (int i = tid; i < M * r; i += kGsThreads) {
    float t = 0.0f;
    for (int z = 0; z < kTSplits; ++z) t += Tpart[(int64_t)z * M * r + i];
    const uint16_t tb = f32_to_bf16(t);
    tl[i] = tb;
    if (blockIdx.x == 0) T_out[i] = tb;
  }
  __syncthreads();   // the level tables (each wave fills entries every wave reads) and T

  // --- the weight stream -----------------------------------------------------
  for (int jr = 0; jr < rgs; ++jr) {
    float acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[i] = 0.0f;
    uint32_t cwl[CW];
#pragma unroll
    for (int q = 0; q < CW; ++q) cwl[q] = cw[q];
    const float scl = sc;
    if (jr + 1 < rgs) load_consts(jr + 1);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      // a_hat of the lane's block (row n; block 2u + g/2 of the slice, or u)
      const int b = PAIR ? 2 * u : u;
      const uint32_t sh = 8u * (uint32_t)(b & 3) + (PAIR ? 8u * (uint32_t)(g >> 1) : 0u);
      const int code = (int)((cwl[b >> 2] >> sh) & 0xffu);
      const float ah = absmax_decode_tab(code, scl, mean, q8);
      const uint4 pw = wu[u % D];
      if (u + D < NU) load_unit(jr, u + D);
      else if (jr + 1 < rgs) load_unit(jr + 1, u + D - NU);
      const uint32_t words[4] = {pw.x, pw.y, pw.z, pw.w};
      f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // byte e of the word: byte address = byte * 256 + 4 * lane
          const uint32_t addr = __builtin_amdgcn_perm(words[j], lane4, 0x0C0C0400u | ((4u + e) << 8));
          o[e] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(tbl) + addr);
        }
        c = mfma_16x16x32(xop[u][j], __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3])), c);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[i] += ah * c[i];
    }
    float* pb = part + jr * PARTW;
    if constexpr (MI == 4) {
      *reinterpret_cast<f32x4_t*>(&pb[(wave * 64 + lane) * 4]) = f32x4_t{acc[0], acc[1 % MI], acc[2 % MI], acc[3 % MI]};
    } else {
      pb[wave * 64 + lane] = acc[0];
    }
  }
  __syncthreads();

  // --- the adapter term and Y (the table's space is free now) --------------
  float* ad = reinterpret_cast<float*>(tbl);                  // (T B^T)[16 jr + row][m]
  if (wave < rgs) {   // wave w: adapter term of row group w, tokens x rows
    f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ch = 0; ch < BCH; ++ch) {
      uint4 tv = make_uint4(0, 0, 0, 0);
      if (col < M && 32 * ch + 8 * g < r) tv = *reinterpret_cast<const uint4*>(tl + col * r + 32 * ch + 8 * g);
      c = mfma_16x16x32(__builtin_bit_cast(bf16x8_t, tv), __builtin_bit_cast(bf16x8_t, bpre[ch]), c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[(16 * wave + col) * kGemvMaxM + 4 * g + i] = c[i];
  }
  __syncthreads();
  for (int i = tid; i < rgs * 16 * M; i += kGsThreads) {
    const int jr = i / (16 * M), m = (i / 16) % M, cc = i % 16;
    const int64_t n = row0 + 16 * jr + cc;
    const float* pb = part + jr * PARTW;
    float base = 0.0f;
    for (int ww = 0; ww < kGsWaves; ++ww) {
      if (MI == 1) {
        for (int h = 0; h < 2; ++h) base += pb[ww * 64 + cc + 32 * h];
      } else if (PAIR) {
        for (int h = 0; h < 2; ++h) base += pb[(ww * 64 + cc + 16 * (2 * h + (m >> 2))) * 4 + (m & 3)];
      } else {
        base += pb[(ww * 64 + cc + 16 * (m >> 2)) * 4 + (m & 3)];
      }
    }
    if (n < N) Y[(int64_t)m * N + n] = f32_to_bf16(base + s * ad[(16 * jr + cc) * kGemvMaxM + m]);
  }
}

// The split kernel's shapes: K of 32, 64 or 128 blocks (S = 4, 8, 16 blocks
// per wave), r <= 64, rows in at most 256 x kGsMaxRG groups of 16.
static int gemv_split_rows(int64_t N, int64_t K, int r) {
  const int64_t Kb = K / kBlock;
  if (Kb != 32 && Kb != 64 && Kb != 128) return 0;
  if (r > 16 * kGsMaxRT || r % 8 != 0) return 0;
  const int64_t groups = (N + 15) / 16;
  const int64_t per = (groups + 255) / 256;       // row groups per workgroup
  if (per > kGsMaxRG) return 0;
  return (int)(per * 16);
}

template <int S, int RT>
static void launch_gemv_split_rt(const uint16_t* X, int M, const NF4Weight& w, const float* Tpart,
                                 const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T,
                                 int rows_wg, hipStream_t st, Span sp) {
  const dim3 grid((unsigned)((w.N + rows_wg - 1) / rows_wg));
  if (M == 1)
    hipExtLaunchKernelGGL((k_gemv_split<S, true, 1, RT>), grid, dim3(kGsThreads), 0, st, sp.start,
                          sp.stop, 0, X, M, w, Tpart, B, r, s, Y, T, rows_wg);
  else if (M <= 8)
    hipExtLaunchKernelGGL((k_gemv_split<S, true, 4, RT>), grid, dim3(kGsThreads), 0, st, sp.start,
                          sp.stop, 0, X, M, w, Tpart, B, r, s, Y, T, rows_wg);
  else
    hipExtLaunchKernelGGL((k_gemv_split<S, false, 4, RT>), grid, dim3(kGsThreads), 0, st, sp.start,
                          sp.stop, 0, X, M, w, Tpart, B, r, s, Y, T, rows_wg);
}

template <int S>
static void launch_gemv_split_s(const uint16_t* X, int M, const NF4Weight& w, const float* Tpart,
                                const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T,
                                int rows_wg, hipStream_t st, Span sp) {
  if (r <= 16) launch_gemv_split_rt<S, 1>(X, M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp);
  else if (r <= 32) launch_gemv_split_rt<S, 2>(X, M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp);
  else launch_gemv_split_rt<S, 4>(X, M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp);
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                       const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T, float* Tpart,
                       hipStream_t st, const uint16_t* Xa, const Timing* tm) {
  if (!Xa) Xa = X;
  hipLaunchKernelGGL(k_lora_down_partial, dim3((r + 31) / 32, kTSplits), dim3(64 * kTWaves), 0, st,
                     Xa, (int)M, w.K, A, r, Tpart);
  // The timed interval is the weight stream (the layer's dominant kernel),
  // recorded by its launch; the T partials before it are a separate, short
  // launch.
  const Span sp = span_of(tm, TK_GEMV);
  const int rows_wg = gemv_split_rows(w.N, w.K, r);
  if (rows_wg > 0) {
    switch (w.K / kBlock) {
      case 32: launch_gemv_split_s<4>(X, (int)M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp); break;
      case 64: launch_gemv_split_s<8>(X, (int)M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp); break;
      default: launch_gemv_split_s<16>(X, (int)M, w, Tpart, B, r, s, Y, T, rows_wg, st, sp); break;
    }
  } else {
    const unsigned grid = (unsigned)((w.N + 63) / 64);
    if ((w.K / kBlock) % (4 * kGemvSS) == 0)
      hipExtLaunchKernelGGL(k_gemv_dma<16>, dim3(grid), dim3(256), 0, st, sp.start, sp.stop, 0, X,
                            (int)M, w, Tpart, B, r, s, Y, T);
    else
      hipExtLaunchKernelGGL(k_gemv_nf4<16>, dim3(grid), dim3(256), 0, st, sp.start, sp.stop, 0, X,
                            (int)M, w, Tpart, B, r, s, Y, T);
  }
  return hipGetLastError();
}

}  // namespace qlk
