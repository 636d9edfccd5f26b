// MFMA tile GEMM for the QLoRA linear layer on gfx950, with operand loaders
// that dequantise NF4 tiles on the fly.
//
//   C[P, Q] = sum_c Aop[p, c] * Bop[q, c]          (phase 1, contraction C1)
//           + sum_j Aop2[p, j] * Bop2[q, j]        (phase 2, the rank-r adapter)
//
// Both operands are staged in LDS as bf16 tiles and fed to
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// The loaders take each operand from its storage form:
//   BF16K   bf16 matrix whose contraction index is contiguous (X, dY, T, U, A)
//   BF16T   bf16 matrix whose contraction index is its row index (B, A for
//           the dX epilogue, X and dY for the adapter gradients, T, U); kept
//           in that orientation in LDS and read with LDS transpose reads
//   NF4K    the NF4 weight for Y = X W^T: rows n, contraction k
//   NF4T    the NF4 weight for dX = dY W: contraction n; decoded in the
//           weight's own orientation and read with transpose reads
// The NF4 loaders compute exactly the dequantised bf16 weight of the
// standalone dequantiser: w_hat = fp32(Q4[nibble] * a_hat), rounded to bf16.
// Each weight tile is decoded once per workgroup into LDS and then shared by
// all of its waves.
//
// Phase 2 is the adapter epilogue fused into the same accumulators:
//   forward  Y  = [X | T] [W_hat | s B]^T          (llm-compass "QLoRA",
//   backward dX = [dY | U] [W_hat ; s A]            方法与公式, the equation)
//
// Workgroups are ordered so that the ones that run on the same XCD (the
// hardware deals workgroup ids round-robin over the 8 XCDs) cover a compact
// block of output tiles and therefore share operand rows in their L2.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kThreads = 256;

constexpr int kPad = 8;   // bf16 elements of padding per LDS row (bank spread)

struct Operand {
  const uint16_t* p;   // bf16 source (unused by NF4 loaders)
  int64_t ld;          // row stride of the SOURCE matrix, in elements
  int rows;            // bound on the operand's row index
  uint32_t bytes;      // size of the source buffer in bytes (< 2^31)
  float scale;         // value multiplier (scaled loaders only)
};

struct GemmArgs {
  Operand a1, b1, a2, b2;
  NF4Weight w;
  int P, Q;
  int c1_len, c1_split, c2_len;
  int tiles_p, tiles_q, group_p;
  void* out;
  int64_t ldo;
  int accumulate;
};

// ------------------------------- loaders -----------------------------------
//
struct LdNone {
  static constexpr bool TR = false;
  struct Regs {};
  __device__ void init(const Operand&, const GemmArgs&, int, int) {}
  __device__ void load(Regs&, const Operand&, const GemmArgs&, int, int) {}
  __device__ void store(const Regs&, const Operand&, uint16_t*, const Dec&) {}
};

__device__ __forceinline__ uint4 scale8(uint4 x, float s) {
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = pack_bf16x2(bf16_to_f32(w[q] & 0xffffu) * s, bf16_to_f32(w[q] >> 16) * s);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// bf16 operand whose contraction index is contiguous: 16-byte chunks.
template <int ROWS, int BK, bool SCALE>
struct LdBF16K {
  static constexpr bool TR = false;
  static constexpr int CPR = BK / 8;
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER_T = CHUNKS / kThreads;
  static_assert(CHUNKS % kThreads == 0, "whole chunks per lane");
  uint32_t voff[PER_T];
  int cc[PER_T];
  int lds_off[PER_T];
  struct Regs { uint4 v[PER_T]; };
  __device__ void init(const Operand& op, const GemmArgs&, int row0, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int r = ch / CPR;
      cc[i] = (ch % CPR) * 8;
      const int row = row0 + r;
      voff[i] = row < op.rows ? (uint32_t)((int64_t)row * op.ld + cc[i]) * 2u : kOOB;
      lds_off[i] = r * (BK + kPad) + cc[i];
    }
  }
  __device__ void load(Regs& R, const Operand& op, const GemmArgs&, int c0, int c_end) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_whole(op.p, op.bytes);
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(c0) * 2u;
#pragma unroll
    for (int i = 0; i < PER_T; ++i)
      R.v[i] = bload128s(rs, c0 + cc[i] < c_end ? voff[i] : kOOB, soff);
  }
  __device__ void store(const Regs& R, const Operand& op, uint16_t* lds, const Dec&) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      uint4 x = R.v[i];
      if (SCALE) x = scale8(x, op.scale);
      *reinterpret_cast<uint4*>(lds + lds_off[i]) = x;
    }
  }
};

// Row stride (elements) of an LDS tile stored contraction-major, [BK][ROWS +
// kPadT]: the pad makes consecutive contraction rows start 32 bytes apart in
// the bank space, so the four rows one 16-lane group reads with a transpose
// read fall in distinct banks.
constexpr int kPadT = 16;

// bf16 operand stored with its contraction index as the row index (source
// [C][R], R contiguous).  The tile is kept in that orientation in LDS,
// [BK][ROWS + kPadT], and the MFMA fragments are read with transpose reads.
template <int ROWS, int BK, bool SCALE>
struct LdBF16T {
  static constexpr bool TR = true;
  static constexpr int CPR = ROWS / 8;               // 16-byte chunks per contraction row
  static constexpr int CHUNKS = BK * CPR;
  static constexpr int PER_T = (CHUNKS + kThreads - 1) / kThreads;
  uint32_t voff[PER_T];
  int cl[PER_T];
  int lds_off[PER_T];
  bool active[PER_T];
  struct Regs { uint4 v[PER_T]; };
  __device__ void init(const Operand& op, const GemmArgs&, int row0, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      active[i] = CHUNKS % kThreads == 0 || ch < CHUNKS;
      const int c = ch / CPR, rr = (ch % CPR) * 8;
      cl[i] = c;
      const int row = row0 + rr;
      voff[i] = (active[i] && row < op.rows) ? (uint32_t)((int64_t)c * op.ld + row) * 2u : kOOB;
      lds_off[i] = c * (ROWS + kPadT) + rr;
    }
  }
  __device__ void load(Regs& R, const Operand& op, const GemmArgs&, int c0, int c_end) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_whole(op.p, op.bytes);
    const uint32_t soff = (uint32_t)((int64_t)__builtin_amdgcn_readfirstlane(c0) * op.ld * 2);
#pragma unroll
    for (int i = 0; i < PER_T; ++i)
      R.v[i] = bload128s(rs, (voff[i] != kOOB && c0 + cl[i] < c_end) ? voff[i] : kOOB, soff);
  }
  __device__ void store(const Regs& R, const Operand& op, uint16_t* lds, const Dec&) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      if (!active[i]) continue;
      uint4 x = R.v[i];
      if (SCALE) x = scale8(x, op.scale);
      *reinterpret_cast<uint4*>(lds + lds_off[i]) = x;
    }
  }
};

// Decode 8 nibbles (one little-endian word, element 2b in the high nibble of
// byte b) into 4 words of packed bf16 in element order:
// w_hat = fp32(Q4[nibble] * a_hat), rounded to bf16.  The nibbles are first
// moved to byte-aligned, x4-scaled positions (two shifts and two masks for
// all eight), so each one is a direct byte offset into the level table.
__device__ __forceinline__ void decode8(uint32_t word, float ah, const float* q4, uint32_t (&o)[4]) {
  const uint32_t hi4 = (word >> 2) & 0x3C3C3C3Cu;   // 4 * high nibble, per byte
  const uint32_t lo4 = (word << 2) & 0x3C3C3C3Cu;   // 4 * low nibble, per byte
  const char* t = reinterpret_cast<const char*>(q4);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float qh = *reinterpret_cast<const float*>(t + ((hi4 >> (8 * b)) & 0xffu));
    const float ql = *reinterpret_cast<const float*>(t + ((lo4 >> (8 * b)) & 0xffu));
    o[b] = pack_bf16x2(qh * ah, ql * ah);
  }
}

// NF4 weight for Y = X W^T: rows n, contraction k; one 64-wide NF4 block per
// K-step, two lanes per row (16 packed bytes = 32 weights each).
template <int ROWS>
struct LdNF4K {
  static constexpr bool TR = false;
  static constexpr int BK = 64;
  static constexpr int WORK = ROWS * 2;
  static constexpr int PER_T = WORK / kThreads;
  static_assert(WORK % kThreads == 0, "whole rows per lane pair");
  uint32_t voff_p[PER_T], voff_c[PER_T], blk0[PER_T];
  float rowmask[PER_T];
  int lds_off[PER_T];
  struct Regs { uint4 p[PER_T]; uint32_t code[PER_T]; float sc[PER_T]; };
  __device__ void init(const Operand&, const GemmArgs& g, int row0, int tid) {
    const int64_t nkb = g.w.K / kBlock;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int t = tid + i * kThreads;
      const int r = t >> 1, half = t & 1;
      const int64_t n = row0 + r;
      const bool ok = n < g.w.N;
      voff_p[i] = ok ? (uint32_t)(n * (g.w.K / 2) + half * 16) : kOOB;
      voff_c[i] = ok ? (uint32_t)(n * nkb) : kOOB;
      blk0[i] = ok ? (uint32_t)(n * nkb) : 0u;
      rowmask[i] = ok ? 1.0f : 0.0f;
      lds_off[i] = r * (BK + kPad) + half * 32;
    }
  }
  __device__ void load(Regs& R, const Operand&, const GemmArgs& g, int c0, int) {
    const uint32_t pbytes = (uint32_t)(g.w.N * (g.w.K / 2)), cbytes = (uint32_t)(g.w.N * (g.w.K / kBlock));
    const __amdgpu_buffer_rsrc_t rp = rsrc_whole(g.w.packed, pbytes);
    const __amdgpu_buffer_rsrc_t rc = rsrc_whole(g.w.codes, cbytes);
    const uint32_t cu = (uint32_t)__builtin_amdgcn_readfirstlane(c0);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      R.p[i] = bload128s(rp, voff_p[i], cu / 2u);
      R.code[i] = bload8s(rc, voff_c[i], cu / kBlock);
      R.sc[i] = g.w.scales[(blk0[i] + (uint32_t)c0 / kBlock) / kDQBlock];
    }
  }
  __device__ void store(const Regs& R, const Operand&, uint16_t* lds, const Dec& d) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const float ah = absmax_decode_tab((int)R.code[i], R.sc[i], d.mean, d.q8) * rowmask[i];
      const uint32_t pw[4] = {R.p[i].x, R.p[i].y, R.p[i].z, R.p[i].w};
      uint4* dst = reinterpret_cast<uint4*>(lds + lds_off[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        decode8(pw[q], ah, d.q4, o);
        dst[q] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

// NF4 weight for dX = dY W: the operand's rows are k (the weight's columns)
// and the contraction runs over n (the weight's rows).  The tile is decoded in
// the weight's own orientation, [64 n][ROWS k + kPadT], exactly like the
// forward loader (16 packed bytes = 32 weights of one row per lane), and the
// MFMA reads it with transpose reads.
template <int ROWS>
struct LdNF4T {
  static constexpr bool TR = true;
  static constexpr int BK = 64;
  static constexpr int PPR = ROWS / 32;               // 32-weight pieces per weight row
  static constexpr int WORK = BK * PPR;
  static constexpr int PER_T = (WORK + kThreads - 1) / kThreads;
  uint32_t voff_p[PER_T], voff_c[PER_T], kb_of[PER_T];
  int nl[PER_T], lds_off[PER_T];
  bool active[PER_T], kok[PER_T];
  struct Regs { uint4 p[PER_T]; uint32_t code[PER_T]; float sc[PER_T]; float mask[PER_T]; };
  __device__ void init(const Operand&, const GemmArgs& g, int row0, int tid) {
    const int64_t nkb = g.w.K / kBlock;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int t = tid + i * kThreads;
      active[i] = WORK % kThreads == 0 || t < WORK;
      const int n = t / PPR, piece = t % PPR;
      const int64_t k = row0 + piece * 32;
      nl[i] = n;
      kok[i] = active[i] && k < g.w.K;
      voff_p[i] = kok[i] ? (uint32_t)(n * (g.w.K / 2) + k / 2) : kOOB;
      voff_c[i] = kok[i] ? (uint32_t)(n * nkb + k / kBlock) : kOOB;
      kb_of[i] = (uint32_t)(kok[i] ? n * nkb + k / kBlock : 0);
      lds_off[i] = n * (ROWS + kPadT) + piece * 32;
    }
  }
  __device__ void load(Regs& R, const Operand&, const GemmArgs& g, int c0, int c_end) {
    const int64_t nkb = g.w.K / kBlock;
    const uint32_t pbytes = (uint32_t)(g.w.N * (g.w.K / 2)), cbytes = (uint32_t)(g.w.N * nkb);
    const __amdgpu_buffer_rsrc_t rp = rsrc_whole(g.w.packed, pbytes);
    const __amdgpu_buffer_rsrc_t rc = rsrc_whole(g.w.codes, cbytes);
    const int64_t cu = __builtin_amdgcn_readfirstlane(c0);
    const uint32_t s0 = (uint32_t)(cu * nkb);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const bool ok = kok[i] && c0 + nl[i] < c_end;
      R.p[i] = bload128s(rp, ok ? voff_p[i] : kOOB, (uint32_t)(cu * (g.w.K / 2)));
      R.code[i] = bload8s(rc, ok ? voff_c[i] : kOOB, s0);
      R.sc[i] = g.w.scales[ok ? (s0 + kb_of[i]) / kDQBlock : 0u];
      R.mask[i] = ok ? 1.0f : 0.0f;
    }
  }
  __device__ void store(const Regs& R, const Operand&, uint16_t* lds, const Dec& d) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      if (!active[i]) continue;
      const float ah = absmax_decode_tab((int)R.code[i], R.sc[i], d.mean, d.q8) * R.mask[i];
      const uint32_t pw[4] = {R.p[i].x, R.p[i].y, R.p[i].z, R.p[i].w};
      uint4* dst = reinterpret_cast<uint4*>(lds + lds_off[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        decode8(pw[q], ah, d.q4, o);
        dst[q] = make_uint4(o[0], o[1], o[2], o[3]);
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
  // room for either orientation of each operand tile
  static constexpr int szk(int rows) { return rows * (BK + kPad); }
  static constexpr int szt(int rows) { return BK * (rows + kPadT); }
  static constexpr int LDSA = szk(BM) > szt(BM) ? szk(BM) : szt(BM);
  static constexpr int LDSB = szk(BN) > szt(BN) ? szk(BN) : szt(BN);
  static constexpr int STAGE = LDSA + LDSB;
  static_assert(WGM * WGN == kThreads / 64, "four waves");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");

  // One MFMA operand fragment: 8 consecutive contraction values for row
  // (lane & 31) of the 32-row slice starting at `row`, k-step `ks`.
  //   !TR: tile [rows][BK + kPad], one 16-byte read.
  //    TR: tile [BK][ROWS + kPadT], two transpose reads of four rows each.
  template <bool TR, int ROWS>
  __device__ static bf16x8_t frag(const uint16_t* tile, int row, int ks, int lane) {
    if (!TR) {
      return *reinterpret_cast<const bf16x8_t*>(tile + (row + (lane & 31)) * (BK + kPad) + ks * 16 +
                                                (lane >> 5) * 8);
    } else {
      const int grp = (lane >> 4) & 3, i = lane & 15;
      const uint16_t* p = tile + (ks * 16 + 8 * (grp >> 1) + (i >> 2)) * (ROWS + kPadT) + row +
                          16 * (grp & 1) + 4 * (i & 3);
      const v4s_t lo = lds_read_tr16(p);
      const v4s_t hi = lds_read_tr16(p + 4 * (ROWS + kPadT));
      typedef short v8s_t __attribute__((ext_vector_type(8)));
      const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // MFMAs over one LDS stage.  The operand fragments of k-step ks+1 are read
  // from LDS before the MFMAs of step ks are issued.
  template <bool ATR, bool BTR>
  __device__ static void compute(const uint16_t* As, const uint16_t* Bs, f32x16_t (&acc)[TM][TN],
                                 int wm, int wn, int lane) {
    bf16x8_t a[2][TM], b[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[0][i] = frag<ATR, BM>(As, wm * WTM + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[0][j] = frag<BTR, BN>(Bs, wn * WTN + j * 32, 0, lane);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cb = ks & 1, nb = cb ^ 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) a[nb][i] = frag<ATR, BM>(As, wm * WTM + i * 32, ks + 1, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[nb][j] = frag<BTR, BN>(Bs, wn * WTN + j * 32, ks + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16(a[cb][i], b[cb][j], acc[i][j]);
    }
  }

  // Distance-1 pipeline: loads for step it+1 are issued before step it is
  // multiplied and land in the other LDS stage after it.
  template <class LA, class LB>
  __device__ static void phase(const GemmArgs& g, const Operand& opa, const Operand& opb, int p0,
                                int q0, int cbeg, int cend, uint16_t* smem, f32x16_t (&acc)[TM][TN],
                                const Dec& d, int tid, int wm, int wn, int lane) {
    const int nk = (cend - cbeg + BK - 1) / BK;
    if (nk <= 0) return;
    LA la;
    LB lb;
    la.init(opa, g, p0, tid);
    lb.init(opb, g, q0, tid);
    typename LA::Regs ra;
    typename LB::Regs rb;
    la.load(ra, opa, g, cbeg, cend);
    lb.load(rb, opb, g, cbeg, cend);
    la.store(ra, opa, smem, d);
    lb.store(rb, opb, smem + LDSA, d);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      uint16_t* cur = smem + (it & 1) * STAGE;
      uint16_t* nxt = smem + ((it + 1) & 1) * STAGE;
      const bool more = it + 1 < nk;
      if (more) {
        la.load(ra, opa, g, cbeg + (it + 1) * BK, cend);
        lb.load(rb, opb, g, cbeg + (it + 1) * BK, cend);
      }
      compute<LA::TR, LB::TR>(cur, cur + LDSA, acc, wm, wn, lane);
      if (more) {
        la.store(ra, opa, nxt, d);
        lb.store(rb, opb, nxt + LDSA, d);
      }
      __syncthreads();
    }
  }

};

// One workgroup of the tile engine: tile index `bx` (walked by tile_coords),
// contraction split `z`; smem holds two stages of this tile shape, q4 / q8
// the decode tables.
template <int BM, int BN, int BK, int WGM, int WGN, class LA1, class LB1, class LA2, class LB2, int EPI>
__device__ __forceinline__ void gemm_block(const GemmArgs& g, int bx, int z, uint16_t* smem,
                                           float* q4, float* q8) {
  using T = Tile<BM, BN, BK, WGM, WGN>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  int tp, tq;
  tile_coords(bx, g.tiles_p, g.tiles_q, g.group_p, tp, tq);
  const int p0 = tp * BM, q0 = tq * BN;
  if (tid < 16) q4[tid] = nf4_level(tid);
  q8[tid] = dq_level(tid);
  Dec d;
  d.q4 = q4;
  d.q8 = q8;
  d.mean = g.w.mean ? g.w.mean[0] : 0.0f;
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
  T::template phase<LA1, LB1>(g, g.a1, g.b1, p0, q0, cbeg, cend, smem, acc, d, tid, wm, wn, lane);
  if (g.c2_len > 0 && z == 0)
    T::template phase<LA2, LB2>(g, g.a2, g.b2, p0, q0, 0, g.c2_len, smem, acc, d, tid, wm, wn, lane);

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

template <int BM, int BN, int BK, int WGM, int WGN, class LA1, class LB1, class LA2, class LB2, int EPI>
__global__ void __launch_bounds__(kThreads) k_gemm(GemmArgs g) {
  using T = Tile<BM, BN, BK, WGM, WGN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];
  __shared__ float q4[16];
  __shared__ float q8[256];
  gemm_block<BM, BN, BK, WGM, WGN, LA1, LB1, LA2, LB2, EPI>(g, blockIdx.x, blockIdx.z, smem, q4, q8);
}

constexpr int kPairBK = 64;   // contraction step of the paired skinny products (kBK below)

// Tile shape and loaders of one tile-engine product, for k_gemm_pair.
template <int BM_, int BN_, class LA_, class LB_>
struct GemmShape {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WGM = (BN == 32) ? 4 : (BM == 32 ? 1 : 2);
  static constexpr int WGN = 4 / WGM;
  using LA = LA_;
  using LB = LB_;
};

// Two independent tile-engine products in one launch (the backward's dA and
// dB partials): blocks [0, blocks1) run the first, the rest the second, with
// (tile, split) = (b mod tiles, b div tiles) of each.  The two share the
// stage buffer, sized for the larger tile.
template <class G1, class G2>
__global__ void __launch_bounds__(kThreads) k_gemm_pair(GemmArgs g1, int blocks1, GemmArgs g2) {
  constexpr int S1 = Tile<G1::BM, G1::BN, kPairBK, G1::WGM, G1::WGN>::STAGE;
  constexpr int S2 = Tile<G2::BM, G2::BN, kPairBK, G2::WGM, G2::WGN>::STAGE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (S1 > S2 ? S1 : S2)];
  __shared__ float q4[16];
  __shared__ float q8[256];
  const int b = blockIdx.x;
  if (b < blocks1) {
    const int tiles = g1.tiles_p * g1.tiles_q;
    gemm_block<G1::BM, G1::BN, kPairBK, G1::WGM, G1::WGN, typename G1::LA, typename G1::LB, LdNone,
               LdNone, EPI_F32_PARTIAL>(g1, b % tiles, b / tiles, smem, q4, q8);
  } else {
    const int c = b - blocks1, tiles = g2.tiles_p * g2.tiles_q;
    gemm_block<G2::BM, G2::BN, kPairBK, G2::WGM, G2::WGN, typename G2::LA, typename G2::LB, LdNone,
               LdNone, EPI_F32_PARTIAL>(g2, c % tiles, c / tiles, smem, q4, q8);
  }
}

// Fixed-order reduction of split partials: out = scale * sum_z part[z],
// summed in the order z = 0, 1, ..., splits - 1.  n is a multiple of 4; one
// thread per four outputs (coalesced 16-byte loads, eight splits in flight).
constexpr int kRedThreads = 64;

// ------------------------------- planning ----------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline int r_tile(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

constexpr int kBK = 64;
static_assert(kBK == kPairBK, "paired products use the engine's contraction step");

// dX tile (rows of dX x columns of dX).
constexpr int kDxBM = 128;
constexpr int kDxBN = 128;

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

FwdPlan plan_fwd(int64_t M, int64_t K, int64_t N, int r, bool nf4) {
  FwdPlan p{};
  p.gemv = M <= kGemvMaxM;
  p.off_T = 0;
  size_t off = align256((size_t)M * r * 2);
  p.off_part = off;
  if (!p.gemv) {
    p.t_splits = 1;   // T in one pass (no partial sums)
  } else {
    p.t_splits = kTSplits;
    off += align256((size_t)kTSplits * M * r * 4);
  }
  p.fwd_kz_len = (nf4 && !p.gemv && fwd_nf4_supported(K)) ? fwd_split_len(M, K, N) : 0;
  p.off_fpart = off;
  if (p.fwd_kz_len > 0) {
    const int64_t splits = (K / kBlock + p.fwd_kz_len - 1) / p.fwd_kz_len;
    off += align256((size_t)splits * M * N * 4);
  }
  // Once 256 x 256 tiles of Y fill the device, dequantising the weight once
  // and running the wide bf16 tile beats decoding it in each of the M / 256
  // token tiles (the two give the same bits).
  p.dequant_fwd = nf4 && !p.gemv && fwd_wide_bf16_fits(M, K, N);
  p.off_wbf16 = off;
  if (p.dequant_fwd) off += align256((size_t)N * K * 2);
  p.bytes = off;
  return p;
}

BwdPlan plan_bwd(int64_t M, int64_t K, int64_t N, int r, bool dx) {
  BwdPlan p{};
  p.off_U = 0;
  p.off_T = align256((size_t)M * r * 2);
  p.off_part = p.off_T + align256((size_t)M * r * 2);
  const int64_t rt = ceil_div(r, r_tile(r));
  p.t_splits = 1;   // T and U in one pass (no partial sums)
  p.u_splits = 1;
  // dA and dB: one pass without partial sums where the shape allows, else
  // split partials over the tokens and a fixed-order reduction.
  p.one_pass_grads = adapter_grads_supported(M, K, N, r);
  if (p.one_pass_grads) {
    p.m_splits_a = p.m_splits_b = 0;
    p.off_part_b = p.off_part;
    p.bytes = p.off_part;
  } else {
    p.m_splits_a = actual_splits(M, choose_splits((int64_t)ceil_div(r, r_tile(r)) * ceil_div(K, 128), M));
    p.m_splits_b = actual_splits(M, choose_splits((int64_t)ceil_div(N, 128) * rt, M));
    p.off_part_b = p.off_part + align256((size_t)p.m_splits_a * r * K * 4);
    p.bytes = p.off_part_b + align256((size_t)p.m_splits_b * N * r * 4);
  }
  // Large M: the dequantised weight (bf16, 2 N K bytes, addressed with 32-bit
  // buffer offsets) is reused by every token tile of the dX kernel.
  p.dequant_dx = dx && M >= kDequantDxMinM && dx_nf4_supported(N) && N * K * 2 < ((int64_t)1 << 31);
  p.off_wbf16 = p.bytes;
  if (p.dequant_dx) p.bytes += align256((size_t)N * K * 2);
  p.dx_kz_len = (dx && dx_nf4_supported(N)) ? dx_split_len(M, K, N) : 0;
  p.off_dxpart = p.bytes;
  if (p.dx_kz_len > 0) {
    const int64_t splits = (N / 64 + p.dx_kz_len - 1) / p.dx_kz_len;
    p.bytes += align256((size_t)splits * M * K * 4);
  }
  return p;
}

// ------------------------------- launchers ---------------------------------

// Number of tile rows walked together: the square root of (tiles per XCD x
// the bytes of a B tile / the bytes of an A tile) balances the two operand
// footprints each XCD keeps in its L2.
int group_for(int tiles_p, int tiles_q, double a_tile_bytes, double b_tile_bytes) {
  const double per_xcd = (double)tiles_p * tiles_q / kXCDs;
  int gsz = (int)(sqrt(per_xcd * b_tile_bytes / a_tile_bytes) + 0.5);
  if (gsz < 1) gsz = 1;
  if (gsz > tiles_p) gsz = tiles_p;
  return gsz;
}

template <int BM, int BN, int BK, class LA1, class LB1, class LA2, class LB2, int EPI>
static hipError_t launch_gemm(GemmArgs g, int splits, double a_tile_bytes, double b_tile_bytes,
                              hipStream_t st) {
  constexpr int WGM = (BN == 32) ? 4 : (BM == 32 ? 1 : 2);
  constexpr int WGN = 4 / WGM;
  g.tiles_p = ceil_div(g.P, BM);
  g.tiles_q = ceil_div(g.Q, BN);
  g.group_p = group_for(g.tiles_p, g.tiles_q, a_tile_bytes, b_tile_bytes);
  dim3 grid(g.tiles_p * g.tiles_q, 1, splits);
  hipLaunchKernelGGL((k_gemm<BM, BN, BK, WGM, WGN, LA1, LB1, LA2, LB2, EPI>), grid, dim3(kThreads),
                     0, st, g);
  return hipGetLastError();
}

// Both split reductions of the backward (dA and dB) in one launch, in the
// fixed order above: blocks [0, blocks of dA) take dA, the rest dB.
__global__ void __launch_bounds__(kRedThreads)
k_reduce_splits2(const float* __restrict__ part_a, int splits_a, int64_t n_a, float* __restrict__ out_a,
                 const float* __restrict__ part_b, int splits_b, int64_t n_b, float* __restrict__ out_b,
                 int blocks_a, float scale) {
  const bool first = (int)blockIdx.x < blocks_a;
  const float* part = first ? part_a : part_b;
  const int splits = first ? splits_a : splits_b;
  const int64_t n4 = (first ? n_a : n_b) / 4;
  float* out = first ? out_a : out_b;
  const int64_t blk = first ? blockIdx.x : blockIdx.x - blocks_a;
  const int64_t i4 = blk * kRedThreads + threadIdx.x;
  if (i4 >= n4) return;
  const float4* p = reinterpret_cast<const float4*>(part) + i4;
  float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
  for (int z = 0; z < splits; ++z) {
    const float4 v = p[(int64_t)z * n4];
    t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
  }
  t.x *= scale; t.y *= scale; t.z *= scale; t.w *= scale;
  reinterpret_cast<float4*>(out)[i4] = t;
}

// `src_rows` x `ld` is the whole source matrix (for its byte size).
static Operand opnd(const uint16_t* p, int64_t ld, int rows, int64_t src_rows, float scale = 1.0f) {
  Operand o;
  o.p = p; o.ld = ld; o.rows = rows; o.scale = scale;
  o.bytes = (uint32_t)(src_rows * ld * 2);
  return o;
}

// The backward's two adapter-gradient products in one launch: dA partials
// (rows j of U^T, columns k of X^T) and dB partials (rows n of dY^T, columns
// j of T^T), both contracting over the M tokens in `splits` slices.
static GemmArgs skinny_args(const Operand& a, const Operand& b, int P, int Q, int64_t C, int splits,
                            float* part, int BM, int BN) {
  GemmArgs g{};
  g.a1 = a; g.b1 = b; g.P = P; g.Q = Q;
  g.c1_len = (int)C;
  g.c1_split = split_len(C, splits);
  g.c2_len = 0;
  g.out = part; g.ldo = Q;
  g.tiles_p = ceil_div(P, BM);
  g.tiles_q = ceil_div(Q, BN);
  g.group_p = group_for(g.tiles_p, g.tiles_q, 1.0, 1.0);
  return g;
}

template <int RT>
static hipError_t skinny_pair_rt(const Operand& aa, const Operand& ba, int Pa, int Qa, int splits_a,
                                 float* part_a, const Operand& ab, const Operand& bb, int Pb, int Qb,
                                 int splits_b, float* part_b, int64_t C, hipStream_t st) {
  using GA = GemmShape<RT, 128, LdBF16T<RT, kBK, false>, LdBF16T<128, kBK, false>>;
  using GB = GemmShape<128, RT, LdBF16T<128, kBK, false>, LdBF16T<RT, kBK, false>>;
  const GemmArgs ga = skinny_args(aa, ba, Pa, Qa, C, splits_a, part_a, GA::BM, GA::BN);
  const GemmArgs gb = skinny_args(ab, bb, Pb, Qb, C, splits_b, part_b, GB::BM, GB::BN);
  const int blocks_a = ga.tiles_p * ga.tiles_q * actual_splits(C, splits_a);
  const int blocks_b = gb.tiles_p * gb.tiles_q * actual_splits(C, splits_b);
  hipLaunchKernelGGL((k_gemm_pair<GA, GB>), dim3((unsigned)(blocks_a + blocks_b)), dim3(kThreads), 0,
                     st, ga, blocks_a, gb);
  return hipGetLastError();
}

static hipError_t skinny_pair(int rt, const Operand& aa, const Operand& ba, int Pa, int Qa,
                              int splits_a, float* part_a, const Operand& ab, const Operand& bb,
                              int Pb, int Qb, int splits_b, float* part_b, int64_t C,
                              hipStream_t st) {
  if (rt == 32)
    return skinny_pair_rt<32>(aa, ba, Pa, Qa, splits_a, part_a, ab, bb, Pb, Qb, splits_b, part_b, C, st);
  if (rt == 64)
    return skinny_pair_rt<64>(aa, ba, Pa, Qa, splits_a, part_a, ab, bb, Pb, Qb, splits_b, part_b, C, st);
  return skinny_pair_rt<128>(aa, ba, Pa, Qa, splits_a, part_a, ab, bb, Pb, Qb, splits_b, part_b, C, st);
}

#define QLK_TRY(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)

// T = X A^T (bf16 [M, r]) in one pass over X.
static hipError_t compute_T(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                            uint16_t* T, hipStream_t st) {
  return launch_rank16(X, M, K, A, false, r, T, st);
}

hipError_t launch_qlora_fwd(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                            const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T_out,
                            void* ws, const FwdPlan& plan, hipStream_t st, const uint16_t* Xa,
                            const Timing* tm) {
  const int64_t K = w.K, N = w.N;
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* T = T_out ? T_out : reinterpret_cast<uint16_t*>(base + plan.off_T);
  float* part = reinterpret_cast<float*>(base + plan.off_part);
  if (!Xa) Xa = X;
  if (plan.gemv && !w.bf16) return launch_gemv(X, M, w, A, B, r, s, Y, T, part, st, Xa, tm);
  if (plan.dequant_fwd && !w.bf16) {
    // T = X A^T next to the dequantisation of the weight rows the wide tile
    // reads, then the wide tile on the copy over the first cw column tiles,
    // and where the last wide round would only part-fill the device, the
    // register-decoded tile over the remaining columns (same bits).
    uint16_t* wb = reinterpret_cast<uint16_t*>(base + plan.off_wbf16);
    const int tw = (int)ceil_div(N, 256);
    const int cw = fwd_nf4_supported(K) ? fwd_wide_columns(M, N) : tw;
    NF4Weight wrows = w;
    wrows.N = (int64_t)cw * 256 < N ? (int64_t)cw * 256 : N;
    QLK_TRY(launch_rank16_and_dequant(Xa, M, K, A, false, r, T, wrows, wb, st,
                                      span_of(tm, TK_FWD_DEQUANT)));
    const Span sp = span_of(tm, TK_FWD_GEMM);
    if (cw == tw) return launch_fwd_wide_bf16(X, M, wb, N, K, T, B, r, s, Y, cw, st, sp);
    QLK_TRY(launch_fwd_wide_bf16(X, M, wb, N, K, T, B, r, s, Y, cw, st, Span{sp.start, nullptr}));
    return launch_fwd_nf4(X, M, w, T, B, r, s, Y, st, nullptr, 0, Span{nullptr, sp.stop}, 2 * cw);
  }
  QLK_TRY(compute_T(Xa, M, K, A, r, T, st));
  // A bf16 base: the dX kernel's forward form.
  if (w.bf16 && dx_nf4_supported(K)) {
    timer_begin(tm, TK_FWD_GEMM, st);
    const hipError_t e = launch_fwd_bf16(X, M, w.bf16, N, K, T, B, r, s, Y, st);
    timer_end(tm, TK_FWD_GEMM, st);
    return e;
  }
  GemmArgs g{};
  g.a1 = opnd(X, K, (int)M, M);
  g.b1 = opnd(nullptr, 0, (int)N, 0);
  g.a2 = opnd(T, r, (int)M, M);
  g.b2 = opnd(B, r, (int)N, N, s);
  g.w = w;
  g.P = (int)M; g.Q = (int)N;
  g.c1_len = (int)K; g.c1_split = (int)K; g.c2_len = r;
  g.out = Y; g.ldo = N; g.accumulate = 0;
  hipError_t e;
  if (fwd_nf4_supported(K)) {
    // timed by the launches themselves
    e = launch_fwd_nf4(X, M, w, T, B, r, s, Y, st,
                       plan.fwd_kz_len ? reinterpret_cast<float*>(base + plan.off_fpart) : nullptr,
                       plan.fwd_kz_len, span_of(tm, TK_FWD_GEMM));
    return e;
  }
  timer_begin(tm, TK_FWD_GEMM, st);
  if (w.bf16) {
    g.b1 = opnd(w.bf16, K, (int)N, N);
    e = launch_gemm<128, 128, kBK, LdBF16K<128, kBK, false>, LdBF16K<128, kBK, false>,
                    LdBF16K<128, kBK, false>, LdBF16K<128, kBK, true>, EPI_BF16>(
        g, 1, 128.0 * K * 2, 128.0 * K * 2, st);
  } else {
    e = launch_gemm<128, 128, kBK, LdBF16K<128, kBK, false>, LdNF4K<128>, LdBF16K<128, kBK, false>,
                    LdBF16K<128, kBK, true>, EPI_BF16>(g, 1, 128.0 * K * 2, 128.0 * K * 0.52, st);
  }
  timer_end(tm, TK_FWD_GEMM, st);
  return e;
}

bool mlp_fwd_fused(int64_t M, int64_t K, int64_t I) {
  return M > kGemvMaxM && fwd_nf4_supported(K) && !fwd_wide_bf16_fits(M, K, I);
}

hipError_t launch_mlp_fwd(const uint16_t* X, int64_t M, const LoraLinear& gate,
                          const LoraLinear& up, uint16_t* G, uint16_t* U, uint16_t* H,
                          uint16_t* Tg, uint16_t* Tu, hipStream_t st) {
  const int64_t K = gate.w.K;
  if (!mlp_fwd_fused(M, K, gate.w.N)) return hipErrorInvalidValue;
  QLK_TRY(compute_T(X, M, K, gate.A, gate.r, Tg, st));
  QLK_TRY(compute_T(X, M, K, up.A, up.r, Tu, st));
  return launch_fwd_gated(X, M, gate.w, Tg, gate.B, gate.r, gate.s, up.w, Tu, up.B, up.r, up.s,
                          G, U, H, st);
}

hipError_t launch_qlora_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const NF4Weight& w,
                            const uint16_t* A, const uint16_t* B, int r, float s,
                            const uint16_t* T, uint16_t* dX, float* dA, float* dB,
                            bool accumulate_dx, void* ws, const BwdPlan& plan, hipStream_t st,
                            const uint32_t* mask, float keep_scale, const Timing* tm) {
  const int64_t K = w.K, N = w.N;
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* U = reinterpret_cast<uint16_t*>(base + plan.off_U);
  float* part = reinterpret_cast<float*>(base + plan.off_part);
  float* part_b = reinterpret_cast<float*>(base + plan.off_part_b);
  const int rt = r_tile(r);
  if (!T) {
    uint16_t* Tw = reinterpret_cast<uint16_t*>(base + plan.off_T);
    QLK_TRY(compute_T(X, M, K, A, r, Tw, st));
    T = Tw;
  }
  // U = dY B (B [N, r] read transposed), in one pass over dY; for large M
  // together with the one-off dequantisation of the weight for dX (one
  // launch, the two run side by side): the dX kernel then runs on the bf16
  // copy (the standalone kernel's arithmetic: the same bits as the in-tile
  // decode), so that the M / 256 token tiles do not each decode the whole
  // weight again.
  NF4Weight wx = w;
  if (dX && !w.bf16 && plan.dequant_dx) {
    uint16_t* wb = reinterpret_cast<uint16_t*>(base + plan.off_wbf16);
    QLK_TRY(launch_rank16_and_dequant(dY, M, N, B, true, r, U, w, wb, st, span_of(tm, TK_DX_DEQUANT)));
    wx.bf16 = wb;
  } else {
    QLK_TRY(launch_rank16(dY, M, N, B, true, r, U, st));
  }
  // dX = dY W_hat + s U A.
  if (dX) {
    GemmArgs g{};
    g.a1 = opnd(dY, N, (int)M, M);
    g.b1 = opnd(nullptr, 0, (int)K, 0);
    g.a2 = opnd(U, r, (int)M, M);
    g.b2 = opnd(A, K, (int)K, r, s);      // transposed load of A [r, K]: rows k, contraction j
    g.w = w;
    g.P = (int)M; g.Q = (int)K;
    g.c1_len = (int)N; g.c1_split = (int)N; g.c2_len = r;
    g.out = dX; g.ldo = K; g.accumulate = accumulate_dx ? 1 : 0;
    hipError_t e;
    const bool own = dx_nf4_supported(N);   // timed by its launches; the others around them
    if (!own) timer_begin(tm, TK_DX_GEMM, st);
    if (own) {
      e = launch_dx_nf4(dY, M, wx, U, A, r, s, dX, accumulate_dx, st, mask, keep_scale,
                        plan.dx_kz_len ? reinterpret_cast<float*>(base + plan.off_dxpart) : nullptr,
                        plan.dx_kz_len, span_of(tm, TK_DX_GEMM));
    } else if (mask) {
      // Tile engine with a dropout mask: the masked adapter term is written
      // (or added) first, then dY W_hat is accumulated on top of it.
      e = launch_dx_adapter_masked(U, A, M, K, r, s, mask, keep_scale, dX, accumulate_dx, st);
      if (e == hipSuccess) {
        g.c2_len = 0;
        g.accumulate = 1;
        if (w.bf16) {
          g.b1 = opnd(w.bf16, K, (int)K, N);
          e = launch_gemm<kDxBM, kDxBN, kBK, LdBF16K<kDxBM, kBK, false>,
                          LdBF16T<kDxBN, kBK, false>, LdBF16K<kDxBM, kBK, false>,
                          LdBF16T<kDxBN, kBK, true>, EPI_BF16>(
              g, 1, (double)kDxBM * N * 2, (double)kDxBN * N * 2, st);
        } else {
          e = launch_gemm<kDxBM, kDxBN, kBK, LdBF16K<kDxBM, kBK, false>,
                          LdNF4T<kDxBN>, LdBF16K<kDxBM, kBK, false>,
                          LdBF16T<kDxBN, kBK, true>, EPI_BF16>(
              g, 1, (double)kDxBM * N * 2, (double)kDxBN * N * 0.52, st);
        }
      }
    } else if (w.bf16) {
      g.b1 = opnd(w.bf16, K, (int)K, N);   // transposed load of W [N, K]: rows k, contraction n
      e = launch_gemm<kDxBM, kDxBN, kBK, LdBF16K<kDxBM, kBK, false>,
                      LdBF16T<kDxBN, kBK, false>, LdBF16K<kDxBM, kBK, false>,
                      LdBF16T<kDxBN, kBK, true>, EPI_BF16>(
          g, 1, (double)kDxBM * N * 2, (double)kDxBN * N * 2, st);
    } else {
      e = launch_gemm<kDxBM, kDxBN, kBK, LdBF16K<kDxBM, kBK, false>,
                      LdNF4T<kDxBN>, LdBF16K<kDxBM, kBK, false>,
                      LdBF16T<kDxBN, kBK, true>, EPI_BF16>(
          g, 1, (double)kDxBM * N * 2, (double)kDxBN * N * 0.52, st);
    }
    if (!own) timer_end(tm, TK_DX_GEMM, st);
    QLK_TRY(e);
  }
  // dA = s U^T X and dB = s dY^T T, both contracting over m.
  if (plan.one_pass_grads) return launch_adapter_grads(U, X, dY, T, M, K, N, r, s, dA, dB, st);
  // Otherwise the partials of both in one launch (rows j of U^T and columns
  // k of X^T, both transposed; rows n of dY^T and columns j of T^T), then
  // their fixed-order sums.
  QLK_TRY(skinny_pair(rt, opnd(U, r, r, M), opnd(X, K, (int)K, M), r, (int)K, plan.m_splits_a, part,
                      opnd(dY, N, (int)N, M), opnd(T, r, r, M), (int)N, r, plan.m_splits_b, part_b,
                      M, st));
  // Both fixed-order split reductions in one launch.
  const int64_t na = (int64_t)r * K, nb = N * r;
  const int blocks_a = (int)((na / 4 + kRedThreads - 1) / kRedThreads);
  const int blocks_b = (int)((nb / 4 + kRedThreads - 1) / kRedThreads);
  hipLaunchKernelGGL(k_reduce_splits2, dim3((unsigned)(blocks_a + blocks_b)), dim3(kRedThreads), 0, st, part,
                     actual_splits(M, plan.m_splits_a), na, dA, part_b, actual_splits(M, plan.m_splits_b),
                     nb, dB, blocks_a, s);
  return hipGetLastError();
}

}  // namespace qlk
