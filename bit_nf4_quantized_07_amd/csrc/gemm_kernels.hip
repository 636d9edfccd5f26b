// MFMA tile GEMM for the QLoRA linear layer on gfx950, with operand loaders
// that dequantise NF4 tiles on the fly.
//
//   C[P, Q] = sum_c Aop[p, c] * Bop[q, c]          (phase 1, contraction C1)
//           + sum_j Aop2[p, j] * Bop2[q, j]        (phase 2, the rank-r adapter)
//
// Both operands are staged in LDS as bf16 tiles [rows][BK + pad], contraction
// contiguous, and fed to v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// The loaders take each operand from its storage form:
//   BF16K   bf16 matrix whose contraction index is contiguous (X, dY, T, U, A)
//   BF16MN  bf16 matrix whose contraction index is the row index; an 8x8
//           register transpose turns it around (B, A^T, X^T, dY^T, T^T, U^T)
//   NF4K    the NF4 weight for Y = X W^T: rows n, contraction k
//   NF4MN   the NF4 weight for dX = dY W: rows k, contraction n (transposed
//           decode)
// The NF4 loaders compute exactly the dequantised bf16 weight of the
// standalone dequantiser: w_hat = fp32(Q4[nibble] * a_hat), rounded to bf16.
//
// Phase 2 is the adapter epilogue fused into the same accumulators:
//   forward  Y  = [X | T] [W_hat | s B]^T          (llm-compass "QLoRA",
//   backward dX = [dY | U] [W_hat ; s A]            方法与公式, the equation)
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kThreads = 256;
constexpr int kPad = 8;   // bf16 elements of padding per LDS row (bank spread)

struct Operand {
  const uint16_t* p;   // bf16 source (unused by NF4 loaders)
  int64_t ld;          // row stride of the SOURCE matrix, in elements
  int rows;            // bound on the operand's row index
  float scale;         // value multiplier (scaled loaders only)
};

struct GemmArgs {
  Operand a1, b1, a2, b2;
  NF4Weight w;
  int P, Q;
  int c1_len, c1_split, c2_len;
  void* out;
  int64_t ldo;
  int accumulate;
};

// ------------------------------- loaders -----------------------------------

struct LdNone {
  __device__ void load(const Operand&, const GemmArgs&, int, int, int, int) {}
  __device__ void store(const Operand&, uint16_t*, int, const float*, float) {}
};

template <int ROWS, int BK, bool SCALE>
struct LdBF16K {
  static constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER_T = (CHUNKS + kThreads - 1) / kThreads;
  uint4 v[PER_T];
  __device__ void load(const Operand& op, const GemmArgs&, int row0, int c0, int c_end, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      v[i] = make_uint4(0, 0, 0, 0);
      if (CHUNKS % kThreads == 0 || ch < CHUNKS) {
        const int r = ch / CPR, cc = (ch % CPR) * 8;
        const int row = row0 + r, c = c0 + cc;
        if (row < op.rows && c < c_end)
          v[i] = *reinterpret_cast<const uint4*>(op.p + (int64_t)row * op.ld + c);
      }
    }
  }
  __device__ void store(const Operand& op, uint16_t* lds, int tid, const float*, float) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      if (CHUNKS % kThreads == 0 || ch < CHUNKS) {
        const int r = ch / CPR, cc = (ch % CPR) * 8;
        uint4 x = v[i];
        if (SCALE) x = scale8(x, op.scale);
        *reinterpret_cast<uint4*>(lds + r * (BK + kPad) + cc) = x;
      }
    }
  }
  __device__ static uint4 scale8(uint4 x, float s) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = pack_bf16x2(bf16_to_f32(w[q] & 0xffffu) * s, bf16_to_f32(w[q] >> 16) * s);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <int ROWS, int BK, bool SCALE>
struct LdBF16MN {
  static constexpr int MR = ROWS / 8, MC = BK / 8, MTS = MR * MC;
  static constexpr int PER_T = (MTS + kThreads - 1) / kThreads;
  uint4 v[PER_T][8];
  __device__ void load(const Operand& op, const GemmArgs&, int row0, int c0, int c_end, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int mt = tid + i * kThreads;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = make_uint4(0, 0, 0, 0);
      if (MTS % kThreads == 0 || mt < MTS) {
        const int rr = mt % MR, cc = mt / MR;
        const int row = row0 + rr * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + cc * 8 + j;
          if (row < op.rows && c < c_end)
            v[i][j] = *reinterpret_cast<const uint4*>(op.p + (int64_t)c * op.ld + row);
        }
      }
    }
  }
  __device__ void store(const Operand& op, uint16_t* lds, int tid, const float*, float) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int mt = tid + i * kThreads;
      if (MTS % kThreads == 0 || mt < MTS) {
        const int rr = mt % MR, cc = mt / MR;
        uint4 o[8];
        transpose8x8_b16(v[i], o);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint4 x = o[j];
          if (SCALE) x = LdBF16K<8, 8, true>::scale8(x, op.scale);
          *reinterpret_cast<uint4*>(lds + (rr * 8 + j) * (BK + kPad) + cc * 8) = x;
        }
      }
    }
  }
};

// Decode 8 nibbles (one little-endian word, element 2b in the high nibble of
// byte b) into 4 words of packed bf16 in element order.
__device__ __forceinline__ void decode8(uint32_t word, float ah, const float* q4, uint32_t (&o)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t byte = (word >> (8 * b)) & 0xffu;
    o[b] = pack_bf16x2(q4[byte >> 4] * ah, q4[byte & 15u] * ah);
  }
}

template <int ROWS>   // contraction tile is fixed at 64 (one NF4 block)
struct LdNF4K {
  static constexpr int BK = 64;
  static constexpr int WORK = ROWS * 2;      // two lanes per row, 16 bytes each
  static constexpr int PER_T = (WORK + kThreads - 1) / kThreads;
  uint4 p[PER_T];
  int code[PER_T];
  float sc[PER_T];
  __device__ void load(const Operand&, const GemmArgs& g, int row0, int c0, int, int tid) {
    const int64_t kb = g.w.K / kBlock;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int t = tid + i * kThreads;
      const int r = t >> 1, half = t & 1;
      const int64_t n = row0 + r;
      code[i] = -1;
      p[i] = make_uint4(0, 0, 0, 0);
      sc[i] = 0.0f;
      if ((WORK % kThreads == 0 || t < WORK) && n < g.w.N) {
        p[i] = *reinterpret_cast<const uint4*>(g.w.packed + n * (g.w.K / 2) + c0 / 2 + half * 16);
        const int64_t blk = n * kb + c0 / kBlock;
        code[i] = g.w.codes[blk];
        sc[i] = g.w.scales[blk / kDQBlock];
      }
    }
  }
  __device__ void store(const Operand&, uint16_t* lds, int tid, const float* q4, float mean) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int t = tid + i * kThreads;
      if (WORK % kThreads == 0 || t < WORK) {
        const int r = t >> 1, half = t & 1;
        uint4* dst = reinterpret_cast<uint4*>(lds + r * (BK + kPad) + half * 32);
        if (code[i] < 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = make_uint4(0, 0, 0, 0);
        } else {
          const float ah = absmax_decode(code[i], sc[i], mean);
          const uint32_t pw[4] = {p[i].x, p[i].y, p[i].z, p[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t o[4];
            decode8(pw[q], ah, q4, o);
            dst[q] = make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  }
};

// Transposed NF4 tile: operand rows are k (the weight's columns), the
// contraction runs over n (the weight's rows).  A lane decodes an 8(n) x KM(k)
// micro-tile and writes it transposed.
template <int ROWS, int BK, int KM>
struct LdNF4MN {
  static constexpr int MR = ROWS / KM, MC = BK / 8, MTS = MR * MC;
  static constexpr int PER_T = (MTS + kThreads - 1) / kThreads;
  static_assert(KM == 4 || KM == 8, "micro-tile width");
  uint32_t p[PER_T][8];
  int code[PER_T][8];
  float sc[PER_T][8];
  __device__ void load(const Operand&, const GemmArgs& g, int row0, int c0, int c_end, int tid) {
    const int64_t kb = g.w.K / kBlock;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int mt = tid + i * kThreads;
      const int rr = mt % MR, cc = mt / MR;
      const int64_t k = row0 + rr * KM;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t n = c0 + cc * 8 + j;
        p[i][j] = 0;
        code[i][j] = -1;
        sc[i][j] = 0.0f;
        if ((MTS % kThreads == 0 || mt < MTS) && k < g.w.K && n < c_end) {
          const uint8_t* src = g.w.packed + n * (g.w.K / 2) + k / 2;
          p[i][j] = (KM == 8) ? *reinterpret_cast<const uint32_t*>(src)
                              : (uint32_t)*reinterpret_cast<const uint16_t*>(src);
          const int64_t blk = n * kb + k / kBlock;
          code[i][j] = g.w.codes[blk];
          sc[i][j] = g.w.scales[blk / kDQBlock];
        }
      }
    }
  }
  __device__ void store(const Operand&, uint16_t* lds, int tid, const float* q4, float mean) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int mt = tid + i * kThreads;
      if (MTS % kThreads == 0 || mt < MTS) {
        const int rr = mt % MR, cc = mt / MR;
        uint4 rows[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t o[4] = {0, 0, 0, 0};
          if (code[i][j] >= 0) {
            const float ah = absmax_decode(code[i][j], sc[i][j], mean);
            if (KM == 8) {
              decode8(p[i][j], ah, q4, o);
            } else {
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                const uint32_t byte = (p[i][j] >> (8 * b)) & 0xffu;
                o[b] = pack_bf16x2(q4[byte >> 4] * ah, q4[byte & 15u] * ah);
              }
            }
          }
          rows[j] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        uint4 cols[8];
        transpose8x8_b16(rows, cols);
#pragma unroll
        for (int kk = 0; kk < KM; ++kk)
          *reinterpret_cast<uint4*>(lds + (rr * KM + kk) * (BK + kPad) + cc * 8) = cols[kk];
      }
    }
  }
};

// ------------------------------- kernel ------------------------------------

enum { EPI_BF16 = 0, EPI_F32_PARTIAL = 1 };

template <int BM, int BN, int BK, int WGM, int WGN>
struct Tile {
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int LDSA = BM * (BK + kPad), LDSB = BN * (BK + kPad);
  static constexpr int STAGE = LDSA + LDSB;
  static_assert(WGM * WGN == kThreads / 64, "four waves");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");

  __device__ static void compute(const uint16_t* As, const uint16_t* Bs, f32x16_t (&acc)[TM][TN],
                                 int wm, int wn, int lane) {
    const int lr = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WTM + i * 32 + lr) * (BK + kPad) + kk + lk);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WTN + j * 32 + lr) * (BK + kPad) + kk + lk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
    }
  }

  template <class LA, class LB>
  __device__ static void phase(const GemmArgs& g, const Operand& opa, const Operand& opb, int p0,
                               int q0, int cbeg, int cend, uint16_t* smem, f32x16_t (&acc)[TM][TN],
                               const float* q4, float mean, int tid, int wm, int wn, int lane) {
    const int nk = (cend - cbeg + BK - 1) / BK;
    if (nk <= 0) return;
    LA la;
    LB lb;
    la.load(opa, g, p0, cbeg, cend, tid);
    lb.load(opb, g, q0, cbeg, cend, tid);
    la.store(opa, smem, tid, q4, mean);
    lb.store(opb, smem + LDSA, tid, q4, mean);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      uint16_t* cur = smem + (it & 1) * STAGE;
      uint16_t* nxt = smem + ((it + 1) & 1) * STAGE;
      const bool more = it + 1 < nk;
      if (more) {
        const int c = cbeg + (it + 1) * BK;
        la.load(opa, g, p0, c, cend, tid);
        lb.load(opb, g, q0, c, cend, tid);
      }
      compute(cur, cur + LDSA, acc, wm, wn, lane);
      if (more) {
        la.store(opa, nxt, tid, q4, mean);
        lb.store(opb, nxt + LDSA, tid, q4, mean);
      }
      __syncthreads();
    }
  }
};

template <int BM, int BN, int BK, int WGM, int WGN, class LA1, class LB1, class LA2, class LB2, int EPI>
__global__ void __launch_bounds__(kThreads) k_gemm(GemmArgs g) {
  using T = Tile<BM, BN, BK, WGM, WGN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];
  __shared__ float q4[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int p0 = blockIdx.y * BM, q0 = blockIdx.x * BN, z = blockIdx.z;
  if (tid < 16) q4[tid] = nf4_level(tid);
  const float mean = g.w.mean ? g.w.mean[0] : 0.0f;
  __syncthreads();

  f32x16_t acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int cbeg = z * g.c1_split;
  const int cend = min(g.c1_len, cbeg + g.c1_split);
  T::template phase<LA1, LB1>(g, g.a1, g.b1, p0, q0, cbeg, cend, smem, acc, q4, mean, tid, wm, wn, lane);
  if (g.c2_len > 0 && z == 0)
    T::template phase<LA2, LB2>(g, g.a2, g.b2, p0, q0, 0, g.c2_len, smem, acc, q4, mean, tid, wm, wn, lane);

  // Output layout of a 32x32 accumulator: lane holds column (lane & 31), rows
  // 8*(v/4) + 4*(lane/32) + (v%4) for v = 0..15.
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int col = q0 + wn * T::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = p0 + wm * T::WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (row < g.P && col < g.Q) {
          const float x = acc[i][j][v];
          if (EPI == EPI_BF16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(g.out) + (int64_t)row * g.ldo + col;
            *o = f32_to_bf16(g.accumulate ? x + bf16_to_f32(*o) : x);
          } else {
            float* o = reinterpret_cast<float*>(g.out) + (int64_t)z * g.P * g.Q + (int64_t)row * g.Q + col;
            *o = x;
          }
        }
      }
    }
}

// Fixed-order reduction of split partials: out = scale * sum_z part[z].
__global__ void __launch_bounds__(256)
k_reduce_splits(const float* __restrict__ part, int splits, int64_t n, float scale,
                float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n + i];
  s *= scale;
  if (out_f32) out_f32[i] = s;
  if (out_bf16) out_bf16[i] = f32_to_bf16(s);
}

// ------------------------- small-M forward (GEMV) ---------------------------
//
// For M <= 16 the layer is bound by streaming the packed weight from HBM.
// One wave owns 16 weight rows and walks all of K; v_mfma_f32_16x16x32_bf16
// multiplies the (zero-padded) activations with the UNSCALED bf16 NF4 levels
// of one 64-block at a time, and the block's a_hat is applied to the 16x16
// partial product (the scale is constant along the block), so the weight is
// never scaled element by element.  Each lane loads 8 contiguous packed bytes
// per block; the four lane groups of a row cover its 32 bytes.
__global__ void __launch_bounds__(256)
k_gemv_nf4(const uint16_t* __restrict__ X, int M, NF4Weight w, const uint16_t* __restrict__ T,
           const uint16_t* __restrict__ B, int r, float s, uint16_t* __restrict__ Y) {
  __shared__ uint32_t lut[256];   // byte -> (level of high nibble, level of low nibble) as bf16
  const int tid = threadIdx.x;
  lut[tid] = pack_bf16x2(nf4_level(tid >> 4), nf4_level(tid & 15));
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t N = w.N, K = w.K;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  if (n0 >= N) return;
  const int g = lane >> 4;
  const int64_t n = n0 + (lane & 15);
  const bool nvalid = n < N;
  const int mrow = lane & 15;
  const bool mvalid = mrow < M;
  const float mean = w.mean[0];
  const int64_t nkb = K / kBlock;
  const uint8_t* prow = w.packed + (nvalid ? n : 0) * (K / 2) + g * 8;
  const uint8_t* crow = w.codes + (nvalid ? n : 0) * nkb;
  const int64_t cbase = (nvalid ? n : 0) * nkb;
  const uint16_t* xrow = X + (int64_t)(mvalid ? mrow : 0) * K + g * 16;

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t kb = 0; kb < nkb; ++kb) {
    uint2 pw = make_uint2(0, 0);
    float ah = 0.0f;
    if (nvalid) {
      pw = *reinterpret_cast<const uint2*>(prow + kb * 32);
      ah = absmax_decode(crow[kb], w.scales[(cbase + kb) / kDQBlock], mean);
    }
    f32x4_t part = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t word = t ? pw.y : pw.x;
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = lut[(word >> (8 * b)) & 0xffu];
      const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
      uint4 xa = make_uint4(0, 0, 0, 0);
      if (mvalid) xa = *reinterpret_cast<const uint4*>(xrow + kb * 64 + t * 8);
      part = mfma_16x16x32(__builtin_bit_cast(bf16x8_t, xa), bw, part);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += ah * part[i];
  }
  // Output layout of a 16x16 accumulator: lane holds column (lane & 15) = the
  // weight row n, rows 4*(lane/16) + i = the token m.  Add the adapter term.
  if (!nvalid) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = g * 4 + i;
    if (m < M) {
      float l = 0.0f;
      for (int j = 0; j < r; ++j)
        l += bf16_to_f32(T[(int64_t)m * r + j]) * bf16_to_f32(B[n * r + j]);
      Y[(int64_t)m * N + n] = f32_to_bf16(acc[i] + s * l);
    }
  }
}

// T = X A^T for M <= 16: one workgroup per adapter row j, fixed-order reduction.
__global__ void __launch_bounds__(256)
k_lora_down_small(const uint16_t* __restrict__ X, int M, int64_t K, const uint16_t* __restrict__ A,
                  int r, uint16_t* __restrict__ T) {
  __shared__ float red[4][16];
  const int j = blockIdx.x, tid = threadIdx.x;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
    const uint4 av = *reinterpret_cast<const uint4*>(A + (int64_t)j * K + k);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < M) {
        const uint4 xv = *reinterpret_cast<const uint4*>(X + (int64_t)m * K + k);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[m] += bf16_to_f32(xw[q] & 0xffffu) * bf16_to_f32(aw[q] & 0xffffu);
          acc[m] += bf16_to_f32(xw[q] >> 16) * bf16_to_f32(aw[q] >> 16);
        }
      }
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][m] = v;
  }
  __syncthreads();
  if (tid < M) {
    const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    T[(int64_t)tid * r + j] = f32_to_bf16(v);
  }
}

// ---------------------------- measurement hook ------------------------------

namespace {
hipEvent_t g_timer_start[TK_COUNT] = {};
hipEvent_t g_timer_stop[TK_COUNT] = {};
}  // namespace

void set_kernel_timer(int kernel, hipEvent_t start, hipEvent_t stop) {
  g_timer_start[kernel] = start;
  g_timer_stop[kernel] = stop;
}
void timer_begin(int kernel, hipStream_t st) {
  if (g_timer_start[kernel]) (void)hipEventRecord(g_timer_start[kernel], st);
}
void timer_end(int kernel, hipStream_t st) {
  if (g_timer_stop[kernel]) (void)hipEventRecord(g_timer_stop[kernel], st);
}

// ------------------------------- planning ----------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline int r_tile(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

constexpr int kGemvMaxM = 16;
constexpr int kBK = 64;

// Split a contraction of length C over `blocks` tiles so that roughly 512
// workgroups run, keeping at least 2 BK-steps per split.
static inline int choose_splits(int64_t blocks, int64_t C) {
  int64_t want = (512 + blocks - 1) / blocks;
  int64_t maxs = C / (2 * kBK);
  if (maxs < 1) maxs = 1;
  if (want > maxs) want = maxs;
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  return (int)want;
}
static inline int split_len(int64_t C, int splits) {
  const int64_t per = (C + splits - 1) / splits;
  return (int)(((per + kBK - 1) / kBK) * kBK);
}
static inline int actual_splits(int64_t C, int splits) {
  return ceil_div(C, split_len(C, splits));
}

FwdPlan plan_fwd(int64_t M, int64_t K, int64_t N, int r) {
  FwdPlan p{};
  p.gemv = M <= kGemvMaxM;
  p.off_T = 0;
  size_t off = align256((size_t)M * r * 2);
  p.off_part = off;
  if (!p.gemv) {
    const int64_t blocks = (int64_t)ceil_div(M, 128) * ceil_div(r, r_tile(r));
    p.t_splits = actual_splits(K, choose_splits(blocks, K));
    off += align256((size_t)p.t_splits * M * r * 4);
  } else {
    p.t_splits = 0;
  }
  p.bytes = off;
  return p;
}

BwdPlan plan_bwd(int64_t M, int64_t K, int64_t N, int r) {
  BwdPlan p{};
  p.off_U = 0;
  p.off_T = align256((size_t)M * r * 2);
  p.off_part = p.off_T + align256((size_t)M * r * 2);
  const int64_t mt = ceil_div(M, 128), rt = ceil_div(r, r_tile(r));
  p.t_splits = actual_splits(K, choose_splits(mt * rt, K));
  p.u_splits = actual_splits(N, choose_splits(mt * rt, N));
  p.m_splits_a = actual_splits(M, choose_splits((int64_t)ceil_div(r, r_tile(r)) * ceil_div(K, 128), M));
  p.m_splits_b = actual_splits(M, choose_splits((int64_t)ceil_div(N, 128) * rt, M));
  size_t part = (size_t)p.t_splits * M * r;
  part = part > (size_t)p.u_splits * M * r ? part : (size_t)p.u_splits * M * r;
  part = part > (size_t)p.m_splits_a * r * K ? part : (size_t)p.m_splits_a * r * K;
  part = part > (size_t)p.m_splits_b * N * r ? part : (size_t)p.m_splits_b * N * r;
  p.bytes = p.off_part + align256(part * 4);
  return p;
}

// ------------------------------- launchers ---------------------------------

template <int BM, int BN, int BK, class LA1, class LB1, class LA2, class LB2, int EPI>
static hipError_t launch_gemm(const GemmArgs& g, int splits, hipStream_t st) {
  constexpr int WGM = (BN == 32) ? 4 : (BM == 32 ? 1 : 2);
  constexpr int WGN = 4 / WGM;
  dim3 grid(ceil_div(g.Q, BN), ceil_div(g.P, BM), splits);
  hipLaunchKernelGGL((k_gemm<BM, BN, BK, WGM, WGN, LA1, LB1, LA2, LB2, EPI>), grid, dim3(kThreads),
                     0, st, g);
  return hipGetLastError();
}

static hipError_t launch_reduce(const float* part, int splits, int64_t n, float scale, float* of,
                                uint16_t* ob, hipStream_t st) {
  hipLaunchKernelGGL(k_reduce_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     splits, n, scale, of, ob);
  return hipGetLastError();
}

static Operand opnd(const uint16_t* p, int64_t ld, int rows, float scale = 1.0f) {
  Operand o;
  o.p = p; o.ld = ld; o.rows = rows; o.scale = scale;
  return o;
}

// C[P, Q] partial products over a split contraction, both operands bf16.
// Akind/Bkind: 0 = contraction contiguous (K-major), 1 = transposed (MN-major).
template <int BM, int BN, int AK, int BKIND>
static hipError_t skinny_partials(const Operand& a, const Operand& b, int P, int Q, int64_t C,
                                  int splits, float* part, hipStream_t st) {
  GemmArgs g{};
  g.a1 = a; g.b1 = b; g.P = P; g.Q = Q;
  g.c1_len = (int)C;
  g.c1_split = split_len(C, splits);
  g.c2_len = 0;
  g.out = part; g.ldo = Q;
  using LA = typename std::conditional<AK == 0, LdBF16K<BM, kBK, false>, LdBF16MN<BM, kBK, false>>::type;
  using LB = typename std::conditional<BKIND == 0, LdBF16K<BN, kBK, false>, LdBF16MN<BN, kBK, false>>::type;
  return launch_gemm<BM, BN, kBK, LA, LB, LdNone, LdNone, EPI_F32_PARTIAL>(g, actual_splits(C, splits), st);
}

// Dispatch on the adapter-rank tile (32, 64 or 128).
template <int AK, int BKIND, bool R_ON_P>
static hipError_t skinny(int rt, const Operand& a, const Operand& b, int P, int Q, int64_t C,
                         int splits, float* part, hipStream_t st) {
  if (R_ON_P) {
    if (rt == 32) return skinny_partials<32, 128, AK, BKIND>(a, b, P, Q, C, splits, part, st);
    if (rt == 64) return skinny_partials<64, 128, AK, BKIND>(a, b, P, Q, C, splits, part, st);
    return skinny_partials<128, 128, AK, BKIND>(a, b, P, Q, C, splits, part, st);
  } else {
    if (rt == 32) return skinny_partials<128, 32, AK, BKIND>(a, b, P, Q, C, splits, part, st);
    if (rt == 64) return skinny_partials<128, 64, AK, BKIND>(a, b, P, Q, C, splits, part, st);
    return skinny_partials<128, 128, AK, BKIND>(a, b, P, Q, C, splits, part, st);
  }
}

#define QLK_TRY(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)

// T = X A^T (bf16 [M, r]) through split partials + fixed-order reduction.
static hipError_t compute_T(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                            int splits, float* part, uint16_t* T, hipStream_t st) {
  QLK_TRY((skinny<0, 0, false>(r_tile(r), opnd(X, K, (int)M), opnd(A, K, r), (int)M, r, K, splits,
                               part, st)));
  return launch_reduce(part, actual_splits(K, splits), M * r, 1.0f, nullptr, T, st);
}

hipError_t launch_qlora_fwd(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                            const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T_out,
                            void* ws, const FwdPlan& plan, hipStream_t st) {
  const int64_t K = w.K, N = w.N;
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* T = T_out ? T_out : reinterpret_cast<uint16_t*>(base + plan.off_T);
  if (plan.gemv) {
    hipLaunchKernelGGL(k_lora_down_small, dim3(r), dim3(256), 0, st, X, (int)M, K, A, r, T);
    QLK_TRY(hipGetLastError());
    const unsigned grid = (unsigned)((N + 63) / 64);
    timer_begin(TK_GEMV, st);
    hipLaunchKernelGGL(k_gemv_nf4, dim3(grid), dim3(256), 0, st, X, (int)M, w, T, B, r, s, Y);
    timer_end(TK_GEMV, st);
    return hipGetLastError();
  }
  float* part = reinterpret_cast<float*>(base + plan.off_part);
  QLK_TRY(compute_T(X, M, K, A, r, plan.t_splits, part, T, st));
  GemmArgs g{};
  g.a1 = opnd(X, K, (int)M);
  g.b1 = opnd(nullptr, 0, (int)N);
  g.a2 = opnd(T, r, (int)M);
  g.b2 = opnd(B, r, (int)N, s);
  g.w = w;
  g.P = (int)M; g.Q = (int)N;
  g.c1_len = (int)K; g.c1_split = (int)K; g.c2_len = r;
  g.out = Y; g.ldo = N; g.accumulate = 0;
  timer_begin(TK_FWD_GEMM, st);
  const hipError_t e = launch_gemm<128, 128, kBK, LdBF16K<128, kBK, false>, LdNF4K<128>,
                                   LdBF16K<128, kBK, false>, LdBF16K<128, kBK, true>, EPI_BF16>(g, 1, st);
  timer_end(TK_FWD_GEMM, st);
  return e;
}

hipError_t launch_qlora_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const NF4Weight& w,
                            const uint16_t* A, const uint16_t* B, int r, float s,
                            const uint16_t* T, uint16_t* dX, float* dA, float* dB,
                            bool accumulate_dx, void* ws, const BwdPlan& plan, hipStream_t st) {
  const int64_t K = w.K, N = w.N;
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* U = reinterpret_cast<uint16_t*>(base + plan.off_U);
  float* part = reinterpret_cast<float*>(base + plan.off_part);
  const int rt = r_tile(r);
  if (!T) {
    uint16_t* Tw = reinterpret_cast<uint16_t*>(base + plan.off_T);
    QLK_TRY(compute_T(X, M, K, A, r, plan.t_splits, part, Tw, st));
    T = Tw;
  }
  // U = dY B: rows m (dY, contraction n contiguous), cols j (B^T: transposed load of B [N, r]).
  QLK_TRY((skinny<0, 1, false>(rt, opnd(dY, N, (int)M), opnd(B, r, r), (int)M, r, N, plan.u_splits,
                               part, st)));
  QLK_TRY(launch_reduce(part, actual_splits(N, plan.u_splits), M * r, 1.0f, nullptr, U, st));
  // dX = dY W_hat + s U A.
  if (dX) {
    GemmArgs g{};
    g.a1 = opnd(dY, N, (int)M);
    g.b1 = opnd(nullptr, 0, (int)K);
    g.a2 = opnd(U, r, (int)M);
    g.b2 = opnd(A, K, (int)K, s);      // transposed load of A [r, K]: rows k, contraction j
    g.w = w;
    g.P = (int)M; g.Q = (int)K;
    g.c1_len = (int)N; g.c1_split = (int)N; g.c2_len = r;
    g.out = dX; g.ldo = K; g.accumulate = accumulate_dx ? 1 : 0;
    timer_begin(TK_DX_GEMM, st);
    const hipError_t e = launch_gemm<128, 128, kBK, LdBF16K<128, kBK, false>, LdNF4MN<128, kBK, 4>,
                                     LdBF16K<128, kBK, false>, LdBF16MN<128, kBK, true>, EPI_BF16>(g, 1, st);
    timer_end(TK_DX_GEMM, st);
    QLK_TRY(e);
  }
  // dA = s U^T X: rows j (U^T, transposed), cols k (X^T, transposed), contraction m.
  QLK_TRY((skinny<1, 1, true>(rt, opnd(U, r, r), opnd(X, K, (int)K), r, (int)K, M, plan.m_splits_a,
                              part, st)));
  QLK_TRY(launch_reduce(part, actual_splits(M, plan.m_splits_a), (int64_t)r * K, s, dA, nullptr, st));
  // dB = s dY^T T: rows n (dY^T), cols j (T^T), contraction m.
  QLK_TRY((skinny<1, 1, false>(rt, opnd(dY, N, (int)N), opnd(T, r, r), (int)N, r, M,
                               plan.m_splits_b, part, st)));
  return launch_reduce(part, actual_splits(M, plan.m_splits_b), N * r, s, dB, nullptr, st);
}

// ------------------------------- SiLU glue ---------------------------------

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }

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
    o[q] = pack_bf16x2(g0 * sigmoidf_(g0) * u0, g1 * sigmoidf_(g1) * u1);
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

}  // namespace qlk
