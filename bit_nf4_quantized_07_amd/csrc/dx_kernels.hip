// Input gradient of the QLoRA linear layer on gfx950:
//
//   dX = dY W_hat + s U A,   U = dY B,   s = alpha / r
//                                   (llm-compass "QLoRA", 方法与公式, the equation,
//                                    differentiated with respect to x)
//
// The contraction runs over n, the weight's row index, so the dequantised
// weight is needed transposed.  One workgroup computes a 256 x 128 tile of
// dX (tokens x input features) with eight waves, two per SIMD: wave w owns
// input features 64 (w % 2) .. +63 of the tile and tokens 64 (w / 2) .. +63,
// four accumulators of v_mfma_f32_32x32x16_bf16, each a 32 (features) x 32
// (tokens) block of dX^T: an MFMA step reads two weight and two dY operands
// for its four MFMAs.  At one wave per SIMD an MFMA and the same wave's
// other instructions barely overlap; the second wave issues its MFMAs while
// the first decodes, reads LDS or waits.
//
//  * dY is staged through LDS exactly like X in the forward kernel: 256 x 64
//    tiles in four buffers, filled by buffer loads that write LDS directly,
//    rows of 128 bytes with the 16-byte pieces XOR-swizzled by (row >> 1) & 7.
//  * The weight tile of a step (64 rows n x 128 features) is decoded once per
//    workgroup: lane L of wave w decodes the 16 weights of row L in features
//    16w .. 16w+15 (8 packed bytes, one 8-bit code, one scale) with the
//    standalone dequantiser's arithmetic
//      a_hat = fp32(fp32(Q8[code] * scale) + mean),
//      w_hat = bf16(fp32(Q4[nibble] * a_hat)),
//    and writes them to LDS in the weight's own orientation.  The MFMA
//    operands are then read with LDS transpose reads (ds_read_b64_tr_b16):
//    eight consecutive rows n of one feature per lane.  The 16-byte pieces of
//    row n are XOR-swizzled by ((n & 3) << 2) | ((n >> 2) & 3), which keeps
//    both the decode stores and the transpose reads free of bank conflicts.
//    Q8[code] is the correctly rounded quotient (code - 127) / 127 (three
//    instructions) and the 16 NF4 levels, repeated every 16 lanes of a
//    register, are fetched with ds_bpermute, so no table occupies LDS.
//  * The weight of step k+1 is decoded during step k into the second weight
//    buffer; raw weight loads run three steps ahead.
//  * The adapter term s U A is a last contraction over r into the same
//    accumulators.  The fp32 tile then goes out through the dY buffers, so
//    that every store instruction writes whole 256-byte row segments of dX.
//    With LoRA dropout on the adapter input the term is accumulated apart,
//    multiplied by mask * 1/(1-p) per element, then added.
//
// NT: the same kernel computes the forward Y = X W_hat^T + s T B^T on a bf16
// weight (the weight dequantised once per call, or a bf16 base).  There the
// contraction runs over the weight's columns, so the weight tile of a step
// (128 rows x 64 columns) has the token tile's shape: it is loaded into LDS
// like the token tile (rows of 128 bytes, the same swizzle) and its MFMA
// operand is read like the token operand, with no transpose.  The adapter
// term takes rows of s B straight from memory.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kDxBM = 256;                 // tokens per tile
constexpr int kDxWaves = 8;
constexpr int kDxWaveK = 64;               // features per wave
constexpr int kDxWaveM = 64;               // tokens per wave
constexpr int kDxBK = 2 * kDxWaveK;        // features per tile
constexpr int kDxStepN = 64;               // contraction (weight rows) per step
constexpr int kDyTile = kDxBM * kDxStepN;  // elements per dY buffer
constexpr int kWTile = kDxStepN * kDxBK;   // elements per weight buffer
constexpr int kDxUnroll = 4;
// s_waitcnt immediates (gfx9 encoding), expcnt not waited on:
// vmcnt <= 7, lgkmcnt <= 4 (end of a step); vmcnt <= 14, lgkmcnt = 0 (prologue).
constexpr int dx_wait(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (lgkm << 8); }

struct DxArgs {
  const uint16_t* dY;   // [M, N] bf16
  int M;
  NF4Weight w;          // N x K
  const uint16_t* U;    // [M, r] bf16
  const uint16_t* A;    // [r, K] bf16
  int r;
  float s;
  uint16_t* dX;         // [M, K] bf16
  int accumulate;
  int tiles_m, tiles_k, group_m;
  int tk_base;          // first feature tile of this launch (a launch can cover the last columns only)
  const uint32_t* mask; // dropout of the adapter input: bit per element of dX, or null
  float keep_scale;     // 1 / (1 - p) for the kept elements
  // Split contraction (fewer tiles than the device has CUs): workgroup
  // b + z tiles takes steps z kz_len .. +kz_len of tile b and writes its fp32
  // partial to part[z] ([M, K]); launch_split_reduce adds the splits.
  // kz_len == 0: one pass, dX written directly.
  float* part;
  int kz_len;
};

struct DxWRegs { uint2 p; uint32_t code; float sc; };

__device__ __forceinline__ int wswz(int n) { return ((n & 3) << 2) | ((n >> 2) & 3); }

// BF16W: the base weight is plain bf16 (g.w.bf16): each step's 64 x 128
// weight tile is copied into LDS by buffer loads that write LDS directly (two
// per wave, the same swizzled layout the decode writes), with nothing to
// decode -- the same kernel with the dequantisation switched off.
template <bool BF16W, bool NT = false>
__global__ void __launch_bounds__(64 * kDxWaves) k_dx_nf4(DxArgs g) {
  static_assert(BF16W || !NT, "the forward form takes a bf16 weight");
  __shared__ __attribute__((aligned(16))) uint16_t dy0[kDyTile];
  __shared__ __attribute__((aligned(16))) uint16_t dy1[kDyTile];
  __shared__ __attribute__((aligned(16))) uint16_t dy2[kDyTile];
  __shared__ __attribute__((aligned(16))) uint16_t dy3[kDyTile];
  __shared__ __attribute__((aligned(16))) uint16_t wt0[kWTile];
  __shared__ __attribute__((aligned(16))) uint16_t wt1[kWTile];
  uint16_t* const dyb[4] = {dy0, dy1, dy2, dy3};
  uint16_t* const wtb[2] = {wt0, wt1};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: LDS bases, offsets
  const int c = lane & 31, h = lane >> 5;
  const int fg = wave & 1, tq = wave >> 1;   // feature half, token quarter

  int tm, tk;
  const int ntiles = g.tiles_m * g.tiles_k;
  const int zsplit = (int)blockIdx.x / ntiles;
  tile_coords((int)blockIdx.x % ntiles, g.tiles_m, g.tiles_k, g.group_m, tm, tk);
  tk += g.tk_base;
  const int m0 = tm * kDxBM;
  const int64_t k0 = (int64_t)tk * kDxBK;
  // N: contraction length; K: output features (dX columns, or Y columns and
  // weight rows in the forward form).
  const int64_t N = NT ? g.w.K : g.w.N, K = NT ? g.w.N : g.w.K, nkb = K / kBlock;
  const int nsteps = (int)(N / kDxStepN);
  // this workgroup's steps (multiples of 4 at both ends)
  const int kz0 = g.kz_len ? zsplit * g.kz_len : 0;
  const int kz1 = g.kz_len ? min(nsteps, kz0 + g.kz_len) : nsteps;
  const float mean = BF16W ? 0.0f : g.w.mean[0];
  const float qlev = nf4_level(lane & 15);   // source of the level lookups

  // dY tile loads: wave w fills rows 32w .. 32w+31, 8 rows per load.
  const uint32_t dybytes = (uint32_t)((int64_t)g.M * N * 2);
  auto swz = [](int row) { return (row >> 1) & 7; };
  uint32_t yoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int piece = (lane & 7) ^ swz(row);
    yoff[i] = m0 + row < g.M ? (uint32_t)(((int64_t)(m0 + row) * N + piece * 8) * 2) : kOOB;
  }
  int yrd[4];   // operand reads: row c, logical piece 2t + h
#pragma unroll
  for (int t = 0; t < 4; ++t) yrd[t] = c * kDxStepN + (((2 * t + h) ^ swz(c)) * 8);
  const __amdgpu_buffer_rsrc_t rdy = rsrc_whole(g.dY, dybytes);
  // dY load i (0..3) of step kb fills rows 32 w + 8 i .. +7 of buffer `buf`.
  auto load_dyi = [&](int i, uint16_t* buf, int kb) {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(kb) * (kDxStepN * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rdy, (__attribute__((address_space(3))) void*)(buf + (32 * wave + 8 * i) * kDxStepN), 16,
        yoff[i], soff, 0, 0);
  };
  auto load_dy = [&](uint16_t* buf, int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_dyi(i, buf, kb);
  };
  // Operand of token block i (32 tokens) of this wave's quarter, MFMA step t.
  auto yfrag = [&](const uint16_t* buf, int i, int t) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(buf + (kDxWaveM * tq + 32 * i) * kDxStepN + yrd[t]);
  };

  // Weight decode: lane L of wave w owns row n = L of the step and features
  // 16w .. 16w+15 of the tile (8 packed bytes of one 64-block).
  const int64_t kcol = k0 + 16 * wave;
  const bool kvalid = kcol < K;
  const uint32_t pbytes = (uint32_t)(N * (K / 2)), cbytes = (uint32_t)(N * nkb);
  const uint32_t sbytes = (uint32_t)(((N * nkb + kDQBlock - 1) / kDQBlock) * 4);
  const uint32_t poff = kvalid ? (uint32_t)((int64_t)lane * (K / 2) + kcol / 2) : kOOB;
  const uint32_t coff = kvalid ? (uint32_t)((int64_t)lane * nkb + kcol / kBlock) : kOOB;
  const __amdgpu_buffer_rsrc_t rp = rsrc_whole(g.w.packed, pbytes);
  const __amdgpu_buffer_rsrc_t rc = rsrc_whole(g.w.codes, cbytes);
  const __amdgpu_buffer_rsrc_t rsc = rsrc_whole(g.w.scales, sbytes);
  // Weight load j (0..2) of rows 64 kb .. 64 kb + 63: packed bytes, code, scale.
  auto load_wj = [&](int j, DxWRegs& R, int kb) {
    const uint32_t row0 = (uint32_t)__builtin_amdgcn_readfirstlane(kb) * kDxStepN;
    if (j == 0) {
      R.p = bload64s(rp, poff, row0 * (uint32_t)(K / 2));
    } else if (j == 1) {
      R.code = bload8s(rc, coff, row0 * (uint32_t)nkb);
    } else {
      const uint32_t blk = row0 * (uint32_t)nkb + coff;
      R.sc = __uint_as_float(bload32(rsc, coff == kOOB ? kOOB : (blk / kDQBlock) * 4u));
    }
  };
  auto load_w = [&](DxWRegs& R, int kb) {
#pragma unroll
    for (int j = 0; j < 3; ++j) load_wj(j, R, kb);
  };
  // bf16 weight tile (rows 64 kb .. +63, features k0 .. k0+127) into LDS:
  // load i of wave w fills rows 8 w + 4 i .. +3 (1 KB); lane L lands at row
  // 8 w + 4 i + L / 16, physical piece L % 16, i.e. logical piece
  // (L % 16) ^ wswz(row).
  const __amdgpu_buffer_rsrc_t rwb = rsrc_whole(g.w.bf16, (uint32_t)(BF16W ? N * K * 2 : 0));
  // NT: load i of wave w fills weight rows 16 w + 8 i .. +7 of the tile
  // (rows of 64 contraction values, 128 bytes); lane L lands at row
  // 16 w + 8 i + L / 8, physical piece L % 8, holding logical piece
  // (L % 8) ^ swz(row) -- the token tile's layout.
  uint32_t wboff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (NT) {
      const int row = 16 * wave + 8 * i + (lane >> 3);
      const int piece = (lane & 7) ^ swz(row);
      const int64_t f = k0 + row;
      wboff[i] = f < K ? (uint32_t)((f * N + piece * 8) * 2) : kOOB;
    } else {
      const int row = 8 * wave + 4 * i + (lane >> 4);
      const int64_t col = k0 + 8 * ((lane & 15) ^ wswz(row));
      wboff[i] = col < K ? (uint32_t)(((int64_t)row * K + col) * 2) : kOOB;
    }
  }
  auto load_wbi = [&](int i, uint16_t* buf, int kb) {
    const uint32_t kbs = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
    const uint32_t soff = NT ? kbs * (kDxStepN * 2) : kbs * kDxStepN * (uint32_t)K * 2u;
    uint16_t* const dst = NT ? buf + (16 * wave + 8 * i) * kDxStepN : buf + (8 * wave + 4 * i) * kDxBK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rwb, (__attribute__((address_space(3))) void*)dst, 16, wboff[i], soff, 0, 0);
  };
  auto word = [](const DxWRegs& R, int t) -> uint32_t { return t == 0 ? R.p.x : R.p.y; };
  // NF4 level of the nibble at bits b .. b+3 of w.  ds_bpermute reads lane
  // addr[7:2] and ignores every other address bit, and qlev repeats the 16
  // levels every 16 lanes, so only addr[5:2] matters: a shift that brings
  // the nibble to bits 2..5 is the whole address computation.
  auto lev = [&](uint32_t w, int b) -> float {
    const uint32_t addr = b >= 2 ? w >> (b - 2) : w << (2 - b);
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)addr, __float_as_int(qlev)));
  };
  auto absmax = [&](const DxWRegs& R) -> float {
#pragma clang fp contract(off)
    const float q = dq_level((int)R.code);
    const float p = q * R.sc;
    return p + mean;
  };
  // Decoded row: two 16-byte pieces (logical 2w, 2w+1) of row `lane`.
  const int wrow = lane;
  auto wstore = [&](uint16_t* buf, int q, uint4 v) {
    const int phys = (2 * wave + q) ^ wswz(wrow);
    *reinterpret_cast<uint4*>(buf + wrow * kDxBK + phys * 8) = v;
  };
  // Transpose-read operand of feature block j (32 features) of the wave's
  // 64: features c, rows 16t + 8h + 0..7.
  const int grp = lane >> 4, gi = lane & 15;
  int wrd[2][4][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int n = 16 * t + 8 * (grp >> 1) + 4 * half + (gi >> 2);
        const int col = kDxWaveK * fg + 32 * j + 16 * (grp & 1) + 4 * (gi & 3);
        const int phys = (col / 8) ^ wswz(n);
        wrd[j][t][half] = n * kDxBK + phys * 8 + (col & 7);
      }
  auto wfrag = [&](const uint16_t* buf, int j, int t) -> bf16x8_t {
    // NT: weight row 64 fg + 32 j + c, whose swizzle equals that of row c
    if constexpr (NT)
      return *reinterpret_cast<const bf16x8_t*>(buf + (kDxWaveK * fg + 32 * j) * kDxStepN + yrd[t]);
    const v4s_t lo = lds_read_tr16(buf + wrd[j][t][0]);
    const v4s_t hi = lds_read_tr16(buf + wrd[j][t][1]);
    typedef short v8s_t __attribute__((ext_vector_type(8)));
    const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };
  auto decode_all = [&](const DxWRegs& R, uint16_t* buf) {
    const float ah = absmax(R);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w = word(R, q);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(lev(w, 8 * e + 4) * ah, lev(w, 8 * e) * ah);
      wstore(buf, q, make_uint4(o[0], o[1], o[2], o[3]));
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // dY(j) is in buffer j % 4 from its load (step j-3) to step j; the raw
  // weight of step j in wr[j % 4] from its load (step j-3) to its decode
  // (step j-1) into weight buffer j % 2, read during step j.
  DxWRegs wr[4];
  bf16x8_t b[2][2];   // dY operands [MFMA step parity][token block]
  __syncthreads();
  if constexpr (BF16W) {
    // W(0) into weight buffer 0, then dY(0..2); W(j+1) is copied during step j.
    load_wbi(0, wtb[0], kz0);
    load_wbi(1, wtb[0], kz0);
#pragma unroll
    for (int j = 0; j < 3; ++j) load_dy(dyb[j], min(kz0 + j, kz1 - 1));
    // W(0), dY(0) and dY(1) arrived (dY(2) may still be in flight): the last
    // slot of step 0 reads the first operands of step 1, which other waves
    // loaded.
    __builtin_amdgcn_s_waitcnt(dx_wait(4, 0));
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      load_dy(dyb[j], min(kz0 + j, kz1 - 1));
      load_w(wr[j], min(kz0 + j, kz1 - 1));
    }
    // Step 0's seven loads must have arrived before its weight is decoded;
    // steps 0 and 1 (step 2's loads may still be in flight) before the
    // barrier publishes dY(0), dY(1) and W(0): the last slot of step 0 reads
    // the first operands of step 1, which other waves loaded.
    __builtin_amdgcn_s_waitcnt(dx_wait(14, 0));
    decode_all(wr[0], wtb[0]);
    __builtin_amdgcn_s_waitcnt(dx_wait(7, 0));
  }
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 2; ++i) b[0][i] = yfrag(dyb[0], i, 0);

  // One step: 16 MFMA slots (t = u / 4 of the 64-row step, token block
  // i = u % 4); the operands of the next MFMA step, the decode of the next
  // weight tile and its two LDS stores are spread over the slots.  The 16
  // level lookups go out in the first four slots and are used from slot 6
  // on, so their latency is covered by MFMAs; the first operands of the next
  // step are read in the last slot, after the decoded weight's stores.
  auto step = [&](auto Pc, int kb) {
    constexpr int P = decltype(Pc)::value;
    const DxWRegs& wdec = wr[(P + 1) % 4];
    DxWRegs& wload = wr[(P + 3) % 4];
    const uint16_t* ycur = dyb[P];
    const uint16_t* ynext = dyb[(P + 1) % 4];
    const uint16_t* wcur = wtb[P % 2];
    uint16_t* wnext = wtb[(P + 1) % 2];

    // This step's 7 loads (for step kb+3) go out one per MFMA slot 0..6, so
    // that the waves released together by the barrier do not queue 56 loads
    // at the address unit before their first MFMA.
    const int kload = min(kb + 3, kz1 - 1);
    uint16_t* const yload = dyb[(P + 3) % 4];
    bf16x8_t a[2][2];   // weight operands [MFMA step parity][feature block]
    a[0][0] = wfrag(wcur, 0, 0);
    a[0][1] = wfrag(wcur, 1, 0);
    float ah = 0.0f;
    float lh[8], ll[8];
    uint32_t o[8];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      // accumulator i: feature block i / 2, token block i % 2
      const int t = u / 4, i = u % 4;
      acc[i] = mfma_32x32x16(a[t & 1][i >> 1], b[t & 1][i & 1], acc[i]);
      if constexpr (BF16W) {
        // W(kb+1) first (it must be complete at this step's end), then dY(kb+3)
        if (u < 2) load_wbi(u, wnext, min(kb + 1, kz1 - 1));
        else if (u < 6) load_dyi(u - 2, yload, kload);
      } else {
        if (u < 4) load_dyi(u, yload, kload);
        else if (u < 7) load_wj(u - 4, wload, kload);
      }
      // operands of MFMA step t+1, one per slot (the other parity)
      if (t < 3) {
        if (i < 2) a[(t + 1) & 1][i] = wfrag(wcur, i, t + 1);
        else b[(t + 1) & 1][i - 2] = yfrag(ycur, i - 2, t + 1);
      }
      if constexpr (!BF16W) {
        if (u < 4) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int v = 2 * u + e;   // byte v % 4 of word v / 4: element 2v high, 2v+1 low
            lh[v] = lev(word(wdec, v / 4), 8 * (v % 4) + 4);
            ll[v] = lev(word(wdec, v / 4), 8 * (v % 4));
          }
        }
        if (u == 1) ah = absmax(wdec);
        if (u >= 6 && u < 14) {
          const int v = u - 6;
          o[v] = pack_bf16x2(lh[v] * ah, ll[v] * ah);
        }
        if (u == 13 || u == 14) {
          const int q = u - 13;
          wstore(wnext, q, make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]));
        }
      }
      if (u == 15) {
#pragma unroll
        for (int j = 0; j < 2; ++j) b[0][j] = yfrag(ynext, j, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Before step kb+1: dY(kb+2) (loaded during step kb-1) in LDS from every
    // wave (at most this step's 7 global loads outstanding; with a bf16
    // weight, at most this step's 4 dY loads, so that W(kb+1) has arrived)
    // and this wave's decoded weight stores done (at most the 2 operand
    // reads of slot 15, issued after them, outstanding), then the barrier.
    __builtin_amdgcn_s_waitcnt(BF16W ? dx_wait(4, 2) : dx_wait(7, 2));
    __builtin_amdgcn_s_barrier();
  };
  for (int kb = kz0; kb < kz1; kb += kDxUnroll) {
    step(std::integral_constant<int, 0>(), kb);
    step(std::integral_constant<int, 1>(), kb + 1);
    step(std::integral_constant<int, 2>(), kb + 2);
    step(std::integral_constant<int, 3>(), kb + 3);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop

  // Adapter term: (s A)^T U^T over r in steps of 16, into the main
  // accumulators, or -- with a dropout mask -- into separate ones that are
  // masked and scaled before they are added.
  const int64_t kw = k0 + kDxWaveK * fg;   // first feature of this wave
  const int mw = m0 + kDxWaveM * tq;       // first token of this wave
  auto adapter_into = [&](f32x16_t (&dst)[4]) {
    for (int r0 = 0; r0 < g.r; r0 += 16) {
      const int rr = r0 + 8 * h;
      bf16x8_t uop[2];   // U rows of the two token blocks
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int m = mw + 32 * ti + c;
        uint4 uv = make_uint4(0, 0, 0, 0);
        if (m < g.M && rr < g.r) uv = *reinterpret_cast<const uint4*>(g.U + (int64_t)m * g.r + rr);
        uop[ti] = __builtin_bit_cast(bf16x8_t, uv);
      }
#pragma unroll
      for (int fi = 0; fi < 2; ++fi) {
        const int64_t kf = kw + 32 * fi + c;   // this lane's feature (operand row)
        uint32_t av[4] = {0u, 0u, 0u, 0u};
        if (NT && kf < K && rr < g.r) {
          // s B, B = g.A here ([K, r]): eight consecutive r of weight row kf
          const uint4 bv = *reinterpret_cast<const uint4*>(g.A + kf * g.r + rr);
          const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            av[q] = pack_bf16x2(bf16_to_f32(bw[q] & 0xffffu) * g.s, bf16_to_f32(bw[q] >> 16) * g.s);
        } else if (!NT && kf < K && rr < g.r) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = bf16_to_f32(g.A[(int64_t)(rr + 2 * q) * K + kf]) * g.s;
            const float hi = bf16_to_f32(g.A[(int64_t)(rr + 2 * q + 1) * K + kf]) * g.s;
            av[q] = pack_bf16x2(lo, hi);
          }
        }
        const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, make_uint4(av[0], av[1], av[2], av[3]));
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) dst[2 * fi + ti] = mfma_32x32x16(afr, uop[ti], dst[2 * fi + ti]);
      }
    }
  };

  // Accumulator i: lane holds token m = mw + 32 (i % 2) + c and features
  // kw + 32 (i / 2) + 8 (v / 4) + 4 h + (v % 4).
  if (zsplit != 0) {
    // the adapter term goes into split 0 only
  } else if (NT || g.mask == nullptr) {
    adapter_into(acc);
  } else {
    f32x16_t ad[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) ad[i][v] = 0.0f;
    adapter_into(ad);
    // A feature block's 32 features start at a multiple of 32 and K % 64 == 0,
    // so a token's 32 mask bits are one word; feature offset 8 (v / 4) + 4 h + v % 4.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mw + 32 * (i & 1) + c;
      const int64_t kw0 = kw + 32 * (i >> 1);
      const uint32_t bits = (m < g.M && kw0 < K) ? g.mask[((int64_t)m * K + kw0) >> 5] : 0u;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int bit = 8 * (v >> 2) + 4 * h + (v & 3);
        acc[i][v] += ((bits >> bit) & 1u) ? ad[i][v] * g.keep_scale : 0.0f;
      }
    }
  }
  if (g.part != nullptr) {
    // split contraction: this split's fp32 partial, four features per store
    float* const pz = g.part + (int64_t)zsplit * g.M * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mw + 32 * (i & 1) + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = kw + 32 * (i >> 1) + 8 * q + 4 * h;
        if (m >= g.M || k >= K) continue;   // K % 8 == 0: a group of four is all in or all out
        *reinterpret_cast<float4*>(pz + (int64_t)m * K + k) =
            make_float4(acc[i][4 * q + 0], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
      }
    }
    return;
  }
  // The fp32 tile goes out through LDS (the dY buffers are free now and hold
  // it exactly: tokens 64 b .. 64 b + 63 in buffer b, rows of 128 features x
  // 4 bytes, the 16-byte pieces of row t XOR-swizzled by t & 31); then each
  // thread takes 8 consecutive features of a token (adds the old dX when
  // accumulating, rounds once) and stores 16 bytes, a wave four whole
  // 256-byte row segments of dX per store instruction.
  __syncthreads();   // every wave's loads into the dY buffers have landed
  {
    float* const st = reinterpret_cast<float*>(tq == 0 ? dy0 : tq == 1 ? dy1 : tq == 2 ? dy2 : dy3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * (i & 1) + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int piece = (16 * fg + 8 * (i >> 1) + 2 * q + h) ^ (row & 31);
        *reinterpret_cast<float4*>(st + row * kDxBK + piece * 4) =
            make_float4(acc[i][4 * q + 0], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // piece 512 j + tid of the tile: token row 32 j + tid / 16, features
    // 8 (tid % 16) .. +7; the row lies in buffer j / 2 at row 32 (j % 2) + tid / 16
    const int rin = 32 * (j & 1) + (tid >> 4), op = tid & 15;
    const int row = 64 * (j >> 1) + rin;
    const float* ld = reinterpret_cast<const float*>(dyb[j >> 1]) + rin * kDxBK;
    const float4 lo = *reinterpret_cast<const float4*>(ld + ((2 * op) ^ (rin & 31)) * 4);
    const float4 hi = *reinterpret_cast<const float4*>(ld + ((2 * op + 1) ^ (rin & 31)) * 4);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const int m = m0 + row;
    const int64_t k = k0 + 8 * op;
    if (m >= g.M || k >= K) continue;   // K % 8 == 0: a piece is all in or all out
    uint4* dst = reinterpret_cast<uint4*>(g.dX + (int64_t)m * K + k);
    if (g.accumulate) {
      const uint4 old = *dst;
      const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += bf16_to_f32(ow[e] & 0xffffu);
        v[2 * e + 1] += bf16_to_f32(ow[e] >> 16);
      }
    }
    *dst = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
  }
}

// ------------------------------------------------------------------------
// Wide tile for large token counts on a bf16 weight (the dequantised copy):
// one workgroup computes a 256 x 256 tile of dX (tokens x features) with
// four waves, one per SIMD, each a 128 x 128 quarter: sixteen accumulators
// of v_mfma_f32_32x32x16_bf16.  Every operand fragment read from LDS feeds
// four MFMAs (two in the 256 x 128 tile above), so the LDS bytes read per
// flop are half those of the eight-wave tile.  The contraction advances 32
// weight rows per step through four LDS stages of 32 KB (a 256 x 32 dY tile
// and a 32 x 256 weight tile each), filled by buffer loads that write LDS
// directly, three steps ahead.
//  * dY tile: rows of 64 bytes, the four 16-byte pieces of row m
//    XOR-swizzled by (m >> 2) & 3: the operand reads (16 rows per bank
//    cycle) are conflict-free.
//  * Weight tile: rows n of 512 bytes (256 features), pieces XOR-swizzled by
//    4 (n & 3), so that the transpose reads (4 rows x 4 pieces per bank
//    cycle) are conflict-free.
//  * The fp32 tile goes out through the stages in four passes of 64 tokens.
// NT: the same tile computes the forward Y = X W_hat^T + s T B^T on the
// dequantised weight ([N, K], rows = outputs): the weight tile is then 256
// weight rows x 32 contraction values, stored and read exactly like the X
// (dY) tile.  The contraction runs in the register-decoded forward's order
// (step 2j holds pieces {0, 1, 4, 5} of 64-block j, step 2j+1 pieces
// {2, 3, 6, 7}; MFMA step t takes logical pieces t and 2 + t), so that Y is
// bit-identical to that kernel's.
constexpr int kWdBM = 256;                    // tokens per tile
constexpr int kWdBK = 256;                    // features per tile
constexpr int kWdStepN = 32;                  // contraction per step
constexpr int kWdYTile = kWdBM * kWdStepN;    // elements per dY stage
constexpr int kWdWTile = kWdStepN * kWdBK;    // elements per weight stage
constexpr int kWdUnroll = 4;                  // steps per loop iteration (= stages)
constexpr int kWdLoads = 8;                   // global loads per wave per step

template <bool NT>
__device__ __forceinline__ void dx_wide_tile(const DxArgs& g) {
  __shared__ __attribute__((aligned(16))) uint16_t y0[kWdYTile];
  __shared__ __attribute__((aligned(16))) uint16_t y1[kWdYTile];
  __shared__ __attribute__((aligned(16))) uint16_t y2[kWdYTile];
  __shared__ __attribute__((aligned(16))) uint16_t y3[kWdYTile];
  __shared__ __attribute__((aligned(16))) uint16_t w0[kWdWTile];
  __shared__ __attribute__((aligned(16))) uint16_t w1[kWdWTile];
  __shared__ __attribute__((aligned(16))) uint16_t w2[kWdWTile];
  __shared__ __attribute__((aligned(16))) uint16_t w3[kWdWTile];
  uint16_t* const yb[4] = {y0, y1, y2, y3};
  uint16_t* const wb[4] = {w0, w1, w2, w3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int fg = wave & 1, tq = wave >> 1;   // feature half, token half

  int tm, tk;
  tile_coords((int)blockIdx.x, g.tiles_m, g.tiles_k, g.group_m, tm, tk);
  tk += g.tk_base;
  const int m0 = tm * kWdBM;
  const int64_t k0 = (int64_t)tk * kWdBK;
  // N: contraction length; K: output features (dX columns, or Y columns and
  // weight rows in the forward form).
  const int64_t N = NT ? g.w.K : g.w.N, K = NT ? g.w.N : g.w.K;
  const int nsteps = (int)(N / kWdStepN);

  // Element offset of logical piece l (8 values) within a step, and the
  // byte offset of step k along a row: natural order for dX, the forward's
  // permuted order for NT.
  auto piece_off = [](int l) { return NT ? 8 * ((l & 1) + 4 * (l >> 1)) : 8 * l; };
  auto step_bytes = [](uint32_t k) {
    return NT ? (k >> 1) * (kBlock * 2) + (k & 1) * 32 : k * (kWdStepN * 2);
  };
  // dY (X) loads: load i of wave w fills rows 64 w + 16 i .. +15 (1 KB); lane
  // L lands at row 64 w + 16 i + L / 4, physical piece L % 4, which holds
  // logical piece (L % 4) ^ ((row >> 2) & 3).
  const __amdgpu_buffer_rsrc_t rdy = rsrc_whole(g.dY, (uint32_t)((int64_t)g.M * N * 2));
  uint32_t yoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 64 * wave + 16 * i + (lane >> 2);
    const int piece = (lane & 3) ^ ((row >> 2) & 3);
    yoff[i] = m0 + row < g.M ? (uint32_t)(((int64_t)(m0 + row) * N + piece_off(piece)) * 2) : kOOB;
  }
  // Weight loads.  dX: load i of wave w fills rows 8 w + 2 i, +1 of the step
  // (1 KB); lane L lands at row 8 w + 2 i + L / 32, physical piece L % 32,
  // which holds logical piece (L % 32) ^ (4 (row & 3)).  NT: as the X loads,
  // for weight rows k0 + 64 w + 16 i + L / 4.
  const __amdgpu_buffer_rsrc_t rw = rsrc_whole(g.w.bf16, (uint32_t)(N * K * 2));
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (NT) {
      const int row = 64 * wave + 16 * i + (lane >> 2);
      const int piece = (lane & 3) ^ ((row >> 2) & 3);
      woff[i] = k0 + row < K ? (uint32_t)(((k0 + row) * N + piece_off(piece)) * 2) : kOOB;
    } else {
      const int row = 8 * wave + 2 * i + (lane >> 5);
      const int64_t col = k0 + 8 * ((lane & 31) ^ (4 * (row & 3)));
      woff[i] = col < K ? (uint32_t)(((int64_t)row * K + col) * 2) : kOOB;
    }
  }
  auto load_j = [&](int j, int buf, int kb) {
    const uint32_t kbs = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
    if (j < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rdy, (__attribute__((address_space(3))) void*)(yb[buf] + (64 * wave + 16 * j) * kWdStepN),
          16, yoff[j], step_bytes(kbs), 0, 0);
    } else if constexpr (NT) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(wb[buf] + (64 * wave + 16 * (j - 4)) * kWdStepN),
          16, woff[j - 4], step_bytes(kbs), 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(wb[buf] + (8 * wave + 2 * (j - 4)) * kWdBK),
          16, woff[j - 4], kbs * kWdStepN * (uint32_t)K * 2u, 0, 0);
    }
  };
  // dY (X) operand of token block i (32 tokens) of this wave's half, MFMA
  // step t: row 128 tq + 32 i + c, logical piece 2 t + h (NT: t + 2 h).
  int yrd[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int l = NT ? t + 2 * h : 2 * t + h;
    yrd[t] = c * kWdStepN + ((l ^ ((c >> 2) & 3)) * 8);
  }
  auto yfrag = [&](int buf, int i, int t) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(yb[buf] + (128 * tq + 32 * i) * kWdStepN + yrd[t]);
  };
  // Weight operand of feature block j (32 features) of this wave's half,
  // MFMA step t: features 128 fg + 32 j + c, rows 16 t + 8 h + 0..7, by two
  // transpose reads of four rows each.
  const int grp = lane >> 4, gi = lane & 15;
  int wrd[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int n = 16 * t + 8 * (grp >> 1) + 4 * half + (gi >> 2);
      const int col = 128 * fg + 16 * (grp & 1) + 4 * (gi & 3);   // + 32 j
      wrd[t][half] = n * kWdBK + (((col >> 3) ^ (4 * (n & 3))) << 3) + (col & 7);
    }
  auto wfrag = [&](int buf, int j, int t) -> bf16x8_t {
    if constexpr (NT)   // weight row 128 fg + 32 j + c of the tile, like the X operand
      return *reinterpret_cast<const bf16x8_t*>(wb[buf] + (128 * fg + 32 * j) * kWdStepN + yrd[t]);
    // Feature block j sets bits 2..3 of the logical piece (0 at j = 0), the
    // bits the swizzle XORs: the physical offset is the j = 0 one XOR 32 j.
    const uint16_t* base = wb[buf];
    const v4s_t lo = lds_read_tr16(base + (wrd[t][0] ^ (32 * j)));
    const v4s_t hi = lds_read_tr16(base + (wrd[t][1] ^ (32 * j)));
    typedef short v8s_t __attribute__((ext_vector_type(8)));
    const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  };

  f32x16_t acc[4][4];   // [feature block][token block]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

  bf16x8_t a[2][4], b[2][4];   // [MFMA step parity][block]
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int j = 0; j < kWdLoads; ++j) load_j(j, s, min(s, nsteps - 1));
  // Steps 0 and 1 in LDS (step 2's loads may still be in flight) before the
  // barrier: the last slots of step 0 read the first operands of step 1.
  __builtin_amdgcn_s_waitcnt(dx_wait(kWdLoads, 0));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) a[0][j] = wfrag(0, j, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[0][i] = yfrag(0, i, 0);

  // One step: 32 MFMA slots (MFMA step t = u / 16, feature block
  // (u % 16) / 4, token block u % 4).  The loads of step kb+3 go out one per
  // slot in slots 0..7; the operands of MFMA step 1 are read in slots 0..7,
  // those of the next step's MFMA step 0 in slots 16..23.
  auto step = [&](auto Pc, int kb) {
    constexpr int P = decltype(Pc)::value;
    constexpr int nxt = (P + 1) % 4, ld = (P + 3) % 4;
    const int kload = min(kb + 3, nsteps - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int t = u / 16, j = (u % 16) / 4, i = u % 4;
      acc[j][i] = mfma_32x32x16(a[t][j], b[t][i], acc[j][i]);
      if (u < kWdLoads) load_j(u, ld, kload);
      if (u < 4) b[1][u] = yfrag(P, u, 1);
      else if (u < 8) a[1][u - 4] = wfrag(P, u - 4, 1);
      else if (u >= 16 && u < 20) b[0][u - 16] = yfrag(nxt, u - 16, 0);
      else if (u >= 20 && u < 24) a[0][u - 20] = wfrag(nxt, u - 20, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Step kb+2's stages (loaded during step kb-1) complete in every wave
    // before step kb+1, which reads them in its last slots: at most this
    // step's loads outstanding, then the barrier.
    __builtin_amdgcn_s_waitcnt(dx_wait(kWdLoads, 0xF));
    __builtin_amdgcn_s_barrier();
  };
  for (int kb = 0; kb < nsteps; kb += kWdUnroll) {
    step(std::integral_constant<int, 0>(), kb);
    step(std::integral_constant<int, 1>(), kb + 1);
    step(std::integral_constant<int, 2>(), kb + 2);
    step(std::integral_constant<int, 3>(), kb + 3);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop

  // Adapter term: (s A)^T U^T over r in steps of 16 into the accumulators
  // (NT: (s B) T^T, B [K, r] row-major).
  const int64_t kw = k0 + 128 * fg;   // first feature of this wave
  const int mw = m0 + 128 * tq;       // first token of this wave
  for (int r0 = 0; r0 < g.r; r0 += 16) {
    const int rr = r0 + 8 * h;
    bf16x8_t uop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mw + 32 * i + c;
      uint4 uv = make_uint4(0, 0, 0, 0);
      if (m < g.M && rr < g.r) uv = *reinterpret_cast<const uint4*>(g.U + (int64_t)m * g.r + rr);
      uop[i] = __builtin_bit_cast(bf16x8_t, uv);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kf = kw + 32 * j + c;
      uint32_t av[4] = {0u, 0u, 0u, 0u};
      if (NT && kf < K && rr < g.r) {
        const uint4 bv = *reinterpret_cast<const uint4*>(g.A + kf * g.r + rr);
        const uint32_t wv[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          av[q] = pack_bf16x2(bf16_to_f32(wv[q] & 0xffffu) * g.s, bf16_to_f32(wv[q] >> 16) * g.s);
      } else if (!NT && kf < K && rr < g.r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_to_f32(g.A[(int64_t)(rr + 2 * q) * K + kf]) * g.s;
          const float hi = bf16_to_f32(g.A[(int64_t)(rr + 2 * q + 1) * K + kf]) * g.s;
          av[q] = pack_bf16x2(lo, hi);
        }
      }
      const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, make_uint4(av[0], av[1], av[2], av[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = mfma_32x32x16(afr, uop[i], acc[j][i]);
    }
  }

  // Accumulator [j][i]: lane holds token mw + 32 i + c and features
  // kw + 32 j + 8 (v / 4) + 4 h + (v % 4).  Four passes of 64 tokens: pass p
  // takes token blocks 2 (p % 2), +1 of the waves with tq == p / 2; row
  // 32 i' + c of the pass (i' = i - 2 (p % 2)) lies in stage y[2 i' + c / 16]
  // at row c % 16, rows of 256 floats whose 16-byte pieces are XOR-swizzled
  // by row % 16.  Then each thread takes 8 consecutive features of a token
  // (adds the old dX when accumulating, rounds once) and stores 16 bytes.
  __syncthreads();   // every wave's loads into the stages have landed
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (tq == p / 2) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * (p % 2) + ii;
        float* const st = reinterpret_cast<float*>(
            (c >> 4) ? (ii ? y3 : y1) : (ii ? y2 : y0)) + (c & 15) * kWdBK;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int piece = (32 * fg + 8 * j + 2 * q + h) ^ (c & 15);
            *reinterpret_cast<float4*>(st + piece * 4) =
                make_float4(acc[j][i][4 * q + 0], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                            acc[j][i][4 * q + 3]);
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // rows 8 e + tid / 32 of the pass (stage e / 2), features 8 (tid % 32) .. +7
      const int row = 8 * e + (tid >> 5), op = tid & 31, rl = row & 15;
      const float* ld = reinterpret_cast<const float*>(yb[e >> 1]) + rl * kWdBK;
      const float4 lo = *reinterpret_cast<const float4*>(ld + ((2 * op) ^ rl) * 4);
      const float4 hi = *reinterpret_cast<const float4*>(ld + ((2 * op + 1) ^ rl) * 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int m = m0 + 128 * (p / 2) + 64 * (p % 2) + row;
      const int64_t k = k0 + 8 * op;
      if (m < g.M && k < K) {   // K % 8 == 0: a piece is all in or all out
        uint4* dst = reinterpret_cast<uint4*>(g.dX + (int64_t)m * K + k);
        if (g.accumulate) {
          const uint4 old = *dst;
          const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] += bf16_to_f32(ow[q] & 0xffffu);
            v[2 * q + 1] += bf16_to_f32(ow[q] >> 16);
          }
        }
        *dst = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7]));
      }
    }
    __syncthreads();
  }
}

// The host pass does not keep a kernel template whose body calls these
// loads from a lambda: one plain kernel per form.
__global__ void __launch_bounds__(256) k_dx_wide(DxArgs g) { dx_wide_tile<false>(g); }
__global__ void __launch_bounds__(256) k_fwd_wide_bf16(DxArgs g) { dx_wide_tile<true>(g); }

// Wide (256-column) tile columns to run before a narrow (128-column) tile
// takes the rest of `width` columns: a wide launch whose last round only
// part-fills the device pays a whole round for it, while narrow tiles, a
// round of which costs about `narrow` of a wide round, can take those
// columns in less.  Both tiles give the same bits.  Returns all the wide
// columns where nothing is gained.
int wide_columns(int tiles_m, int64_t width, double narrow) {
  const int tw = (int)((width + 255) / 256);
  auto rounds = [](int64_t tiles) { return (double)((tiles + kCUs - 1) / kCUs); };
  double best = rounds((int64_t)tiles_m * tw);
  int best_cw = tw;
  for (int cw = tw - 1; cw >= 1 && cw >= tw - 64; --cw) {
    const int64_t nt = (width - 256 * (int64_t)cw + 127) / 128;
    const double cost = rounds((int64_t)tiles_m * cw) + narrow * rounds(tiles_m * nt) + 0.02;
    if (cost < best) {
      best = cost;
      best_cw = cw;
    }
  }
  return best_cw;
}
// A narrow round over a wide round (same contraction): the eight-wave dX
// tile and the register-decoded forward tile, measured.
constexpr double kNarrowRound = 0.6;

// The wide tile pays when its tiles alone fill the device.
static bool dx_wide_fits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + kWdBM - 1) / kWdBM) * ((K + kWdBK - 1) / kWdBK);
  return tiles >= 256 && N % (kWdStepN * kWdUnroll) == 0 && N * K * 2 < ((int64_t)1 << 31) &&
         M * N * 2 < ((int64_t)1 << 31);
}

bool dx_nf4_supported(int64_t N) { return N % (kDxStepN * kDxUnroll) == 0; }

hipError_t launch_dx_nf4(const uint16_t* dY, int64_t M, const NF4Weight& w, const uint16_t* U,
                         const uint16_t* A, int r, float s, uint16_t* dX, bool accumulate,
                         hipStream_t st, const uint32_t* mask, float keep_scale, float* part,
                         int kz_len, Span sp) {
  if (!dx_nf4_supported(w.N)) return hipErrorInvalidValue;
  DxArgs g{};
  g.dY = dY; g.M = (int)M; g.w = w; g.U = U; g.A = A; g.r = r; g.s = s; g.dX = dX;
  g.accumulate = accumulate ? 1 : 0;
  g.mask = mask; g.keep_scale = keep_scale;
  g.tiles_m = (int)((M + kDxBM - 1) / kDxBM);
  g.tiles_k = (int)((w.K + kDxBK - 1) / kDxBK);
  g.group_m = group_for(g.tiles_m, g.tiles_k, (double)kDxBM * w.N * 2,
                        (double)kDxBK * w.N * (w.bf16 ? 2.0 : 0.52));
  if (w.bf16 && mask == nullptr && dx_wide_fits(M, w.N, w.K)) {
    // wide tiles over the first cw feature columns, the eight-wave tile over
    // the rest (same bits)
    const int tm_n = (int)((M + kWdBM - 1) / kWdBM);
    const int tw = (int)((w.K + kWdBK - 1) / kWdBK);
    const int cw = wide_columns(tm_n, w.K, kNarrowRound);
    DxArgs gw = g;
    gw.tiles_m = tm_n;
    gw.tiles_k = cw;
    gw.group_m = group_for(gw.tiles_m, gw.tiles_k, (double)kWdBM * w.N * 2, (double)kWdBK * w.N * 2);
    hipExtLaunchKernelGGL(k_dx_wide, dim3(gw.tiles_m * gw.tiles_k), dim3(256), 0, st, sp.start,
                          cw == tw ? sp.stop : nullptr, 0, gw);
    if (cw == tw) return hipGetLastError();
    g.tk_base = cw * (kWdBK / kDxBK);
    g.tiles_k = (int)((w.K - (int64_t)cw * kWdBK + kDxBK - 1) / kDxBK);
    g.group_m = group_for(g.tiles_m, g.tiles_k, (double)kDxBM * w.N * 2, (double)kDxBK * w.N * 2);
    hipExtLaunchKernelGGL(k_dx_nf4<true>, dim3(g.tiles_m * g.tiles_k), dim3(64 * kDxWaves), 0, st,
                          nullptr, sp.stop, 0, g);
    return hipGetLastError();
  }
  const int nsteps = (int)(w.N / kDxStepN);
  const int splits = (part != nullptr && kz_len > 0) ? (nsteps + kz_len - 1) / kz_len : 1;
  if (splits > 1) {
    g.part = part;
    g.kz_len = kz_len;
  }
  const dim3 grid(g.tiles_m * g.tiles_k * splits);
  hipEvent_t stop = splits > 1 ? nullptr : sp.stop;
  if (w.bf16)
    hipExtLaunchKernelGGL(k_dx_nf4<true>, grid, dim3(64 * kDxWaves), 0, st, sp.start, stop, 0, g);
  else
    hipExtLaunchKernelGGL(k_dx_nf4<false>, grid, dim3(64 * kDxWaves), 0, st, sp.start, stop, 0, g);
  if (splits > 1) return launch_split_reduce(part, splits, M * w.K, dX, accumulate, st, sp.stop);
  return hipGetLastError();
}

int dx_split_len(int64_t M, int64_t K, int64_t N) {
  const int64_t nsteps = N / kDxStepN;
  const int64_t tiles = ((M + kDxBM - 1) / kDxBM) * ((K + kDxBK - 1) / kDxBK);
  if (tiles >= 128 || nsteps < 2 * kDxUnroll) return 0;   // two splits do not pay for the partials
  int64_t splits = 256 / tiles;
  if (splits > nsteps / kDxUnroll) splits = nsteps / kDxUnroll;
  if (splits < 2) return 0;
  const int64_t per = (nsteps + splits - 1) / splits;
  return (int)(((per + kDxUnroll - 1) / kDxUnroll) * kDxUnroll);
}

// The forward form of the wide tile: 256 x 256 tiles of Y that alone fill
// the device, K in whole 64-blocks and steps of four, 32-bit offsets.
bool fwd_wide_bf16_fits(int64_t M, int64_t K, int64_t N) {
  const int64_t tiles = ((M + kWdBM - 1) / kWdBM) * ((N + kWdBK - 1) / kWdBK);
  return tiles >= 256 && K % (kWdStepN * kWdUnroll) == 0 && N * K * 2 < ((int64_t)1 << 31) &&
         M * K * 2 < ((int64_t)1 << 31);
}

int fwd_wide_columns(int64_t M, int64_t N) {
  return wide_columns((int)((M + kWdBM - 1) / kWdBM), N, kNarrowRound);
}

hipError_t launch_fwd_wide_bf16(const uint16_t* X, int64_t M, const uint16_t* wb, int64_t N,
                                int64_t K, const uint16_t* T, const uint16_t* B, int r, float s,
                                uint16_t* Y, int cols, hipStream_t st, Span sp) {
  if (!fwd_wide_bf16_fits(M, K, N) || cols < 1 || (int64_t)cols * kWdBK > N + kWdBK - 1)
    return hipErrorInvalidValue;
  DxArgs g{};
  g.dY = X; g.M = (int)M; g.U = T; g.A = B; g.r = r; g.s = s; g.dX = Y;
  g.w.N = N; g.w.K = K; g.w.bf16 = wb;
  g.accumulate = 0;
  g.mask = nullptr; g.keep_scale = 1.0f;
  g.tiles_m = (int)((M + kWdBM - 1) / kWdBM);
  g.tiles_k = cols;
  g.group_m = group_for(g.tiles_m, g.tiles_k, (double)kWdBM * K * 2, (double)kWdBK * K * 2);
  hipExtLaunchKernelGGL(k_fwd_wide_bf16, dim3(g.tiles_m * g.tiles_k), dim3(256), 0, st, sp.start,
                        sp.stop, 0, g);
  return hipGetLastError();
}

// Forward on a bf16 weight wb ([N, K]): Y = X wb^T + s T B^T.
hipError_t launch_fwd_bf16(const uint16_t* X, int64_t M, const uint16_t* wb, int64_t N, int64_t K,
                           const uint16_t* T, const uint16_t* B, int r, float s, uint16_t* Y,
                           hipStream_t st) {
  if (!dx_nf4_supported(K)) return hipErrorInvalidValue;
  DxArgs g{};
  g.dY = X; g.M = (int)M; g.U = T; g.A = B; g.r = r; g.s = s; g.dX = Y;
  g.w.N = N; g.w.K = K; g.w.bf16 = wb;
  g.accumulate = 0;
  g.mask = nullptr; g.keep_scale = 1.0f;
  g.tiles_m = (int)((M + kDxBM - 1) / kDxBM);
  g.tiles_k = (int)((N + kDxBK - 1) / kDxBK);
  g.group_m = group_for(g.tiles_m, g.tiles_k, (double)kDxBM * K * 2, (double)kDxBK * K * 2);
  hipLaunchKernelGGL((k_dx_nf4<true, true>), dim3(g.tiles_m * g.tiles_k), dim3(64 * kDxWaves), 0, st, g);
  return hipGetLastError();
}

}  // namespace qlk
