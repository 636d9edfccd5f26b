// Forward of the QLoRA linear layer for more than 16 tokens, on gfx950:
//
//   Y = X W_hat^T + s T B^T,   T = X A^T,   s = alpha / r
//                                   (llm-compass "QLoRA", 方法与公式, the equation)
//
// One workgroup computes a 256 x 128 tile of Y (tokens x weight rows) with
// four waves; wave w owns weight rows 32w .. 32w+31 of the tile and all 256
// tokens: eight accumulators of v_mfma_f32_32x32x16_bf16, each computing a
// 32 (weight rows) x 32 (tokens) block of Y^T.
//
//  * X is staged through LDS, one 256 x 64 tile per K-step, in four
//    buffers, by buffer loads that write LDS directly (no registers, no LDS
//    store instructions): X(k+3) is in flight while X(k) is multiplied, and
//    the first MFMA operands of step k+1 are read from the already complete
//    X(k+1) before the barrier that ends step k, so no step starts by
//    waiting on LDS.  Rows are 128 bytes; the 16-byte pieces of row r are
//    stored XOR-swizzled by (r >> 1) & 7, which makes the operand reads
//    (16 rows x 16 bytes per bank cycle) conflict-free.
//  * The NF4 weight never goes through LDS: each lane loads the 16 packed
//    bytes (32 weights) of its weight row that its half of the MFMA operand
//    covers, and decodes them straight into the bf16 MFMA operand; the 8-bit
//    codes of four consecutive blocks come in one 4-byte load, with their
//    shared second-level scale, once every four steps.  Every weight is
//    decoded once.
//    The decode is the standalone dequantiser's arithmetic:
//      a_hat = fp32(fp32(Q8[code] * scale) + mean),
//      w_hat = bf16(fp32(Q4[nibble] * a_hat)),
//    with the fp32 levels in LDS as a 256-entry table of pairs: entry b
//    holds the levels of the high and the low nibble of packed byte b, so
//    one 8-byte read (address: the byte, extracted and shifted) gives both
//    weights of a byte.  The NF4 codes are equiprobable, so the 64 lanes of
//    a read hit the table's banks at random; on the 2048-token layer that
//    cost less than the byte permute and the second read per byte of a
//    16-entry table (69.5 against 72.8 us).
//  * Inside a 64-block the contraction order is permuted so that a lane's 32
//    weights are contiguous in memory: at MFMA step t (0..3) lane half h
//    covers k = 32h + 8t .. 32h + 8t + 7, for X and for the weight alike.
//  * Each K-step is a fixed schedule of 32 MFMA slots; the LDS reads of the
//    decode table are issued 16 slots before their values are used, and the
//    operand reads of MFMA step t+1 during step t.  Global loads of X and of
//    the weight run three K-steps ahead.
//  * The adapter term s T B^T is a last contraction over r into the same
//    accumulators (the up-projection fused into the base GEMM).
//  * The accumulator layout gives each lane four consecutive weight rows of
//    one token (8 bytes of Y); the finished tile goes out through LDS so that
//    every store instruction writes whole 256-byte row segments of Y.
//
// Gated variant (the fused gate/up projections of a SiLU-gated MLP): each
// wave's weight rows come from one weight, so waves 0-1 take 64 rows of the
// gate weight and waves 2-3 the same 64 rows of the up weight, each with its
// own NF4 constants and adapter.  After the main loop the up waves pass their
// bf16 results through LDS to the gate waves, which write
// H = silu(G) U (the elementwise kernel's arithmetic on the same bf16 G and
// U); G and U are written too, for the backward.
#include "device_common.h"
#include "kernels.h"

namespace qlk {

constexpr int kFwdBM = 256;                    // tokens per tile
constexpr int kFwdWaveN = 32;                  // weight rows per wave
constexpr int kFwdBN = 4 * kFwdWaveN;          // weight rows per tile
constexpr int kXRow = kBlock;                  // LDS row of the X tile (elements, swizzled)
constexpr int kXTile = kFwdBM * kXRow;         // elements per X buffer
constexpr int kXBufs = 4;
// s_waitcnt immediates (gfx9 encoding), expcnt not waited on: vmcnt <= the
// loads of one step, lgkmcnt not waited on (end of a step); vmcnt <= the
// loads of two steps, lgkmcnt = 0 (end of the prologue).
constexpr int wait_vm(int n, int lgkm) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (lgkm << 8); }
constexpr int kFwdUnroll = 4;                  // K-steps per loop iteration (register sets)

struct FwdArgs {
  const uint16_t* X;
  int M;
  NF4Weight w;
  const uint16_t* T;    // [M, r] bf16
  const uint16_t* B;    // [N, r] bf16
  int r;
  float s;
  uint16_t* Y;
  int tiles_m, tiles_n, group_m;
  int tn_base;          // first column tile of this launch (a launch can cover the last columns only)
  // gated variant: w/T/B/r/s/Y are the gate projection's (Y = G), these the
  // up projection's (Y2 = U); H = silu(G) U.
  NF4Weight w2;
  const uint16_t* T2;
  const uint16_t* B2;
  int r2;
  float s2;
  uint16_t* Y2;
  uint16_t* H;
  // Split contraction (fewer tiles than the device has CUs): workgroup
  // b + z tiles takes K-steps z kz_len .. +kz_len of tile b and writes its
  // fp32 partial to part[z] ([M, N]); launch_split_reduce adds the splits.
  // kz_len == 0: one pass over K, Y written directly.
  float* part;
  int kz_len;
};

struct FwdWRegs { uint4 p; };   // NF4: 32 packed weights
struct FwdBFrag { uint32_t d[4][4]; };   // [MFMA step][dword]

__device__ __forceinline__ bf16x8_t as_frag(const uint32_t (&d)[4]) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(d[0], d[1], d[2], d[3]));
}

template <bool GATED = false>
__global__ void __launch_bounds__(256) k_fwd_nf4(FwdArgs g) {
  using WRegs = FwdWRegs;
  // Global loads per step: 8 of X and the packed weights, plus, once every
  // four steps (P == 1), the codes and the scale of the next four blocks.
  constexpr int kLoads = 9;
  constexpr int kRunLoads = 2;
  // Tables first (low LDS addresses fit the instructions' offset field),
  // then the X buffers as four separate objects, so that the compiler can
  // tell that a load into one buffer does not alias reads of another.
  __shared__ __attribute__((aligned(64))) float q8[256];
  __shared__ __attribute__((aligned(64))) float2 q44[256];   // byte -> (level of its high nibble, of its low)
  __shared__ __attribute__((aligned(16))) uint16_t xs0[kXTile];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[kXTile];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[kXTile];
  __shared__ __attribute__((aligned(16))) uint16_t xs3[kXTile];
  uint16_t* const xbuf[kXBufs] = {xs0, xs1, xs2, xs3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: LDS bases, offsets
  const int c = lane & 31, h = lane >> 5;
  q8[tid] = dq_level(tid);
  q44[tid] = make_float2(nf4_level(tid >> 4), nf4_level(tid & 15));

  int tm, tn;
  const int ntiles = g.tiles_m * g.tiles_n;
  const int zsplit = (int)blockIdx.x / ntiles;
  tile_coords((int)blockIdx.x % ntiles, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  tn += g.tn_base;
  const int m0 = tm * kFwdBM;
  // This wave's weight (the up weight for waves 2-3 of the gated variant).
  const bool upw = GATED && wave >= 2;
  const NF4Weight W = upw ? g.w2 : g.w;
  const int64_t K = W.K, N = W.N, nkb = K / kBlock;
  const int nk = (int)nkb;
  // this workgroup's K-steps (multiples of 4 at both ends)
  const int kz0 = g.kz_len ? zsplit * g.kz_len : 0;
  const int kz1 = g.kz_len ? min(nk, kz0 + g.kz_len) : nk;
  const float mean = W.mean[0];

  // X tile loads: wave w, load i fills rows 64 w + 8 i .. +7 (1 KB of LDS);
  // lane L lands at LDS offset 16 L, i.e. row 64 w + 8 i + L / 8, physical
  // piece L % 8, which holds logical piece (L % 8) ^ swz(row).
  const uint32_t xbytes = (uint32_t)((int64_t)g.M * K * 2);
  auto swz = [](int row) { return (row >> 1) & 7; };
  uint32_t xoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const int piece = (lane & 7) ^ swz(row);
    xoff[i] = m0 + row < g.M ? (uint32_t)(((int64_t)(m0 + row) * K + piece * 8) * 2) : kOOB;
  }
  // Operand reads: row 32 i + c, logical piece 4 h + t -> physical.
  int xrd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) xrd[t] = c * kXRow + (((4 * h + t) ^ swz(c)) * 8);
  // Weight rows of this wave (gated: 64 rows of each weight per tile).
  const int64_t nw0 = GATED ? (int64_t)tn * (kFwdBN / 2) + (wave & 1) * kFwdWaveN
                            : (int64_t)tn * kFwdBN + wave * kFwdWaveN;
  const int64_t nrow = nw0 + c;
  const bool nvalid = nrow < N;
  const uint32_t pbytes = (uint32_t)(N * (K / 2)), cbytes = (uint32_t)(N * nkb);
  const uint32_t sbytes = (uint32_t)(((N * nkb + kDQBlock - 1) / kDQBlock) * 4);
  const uint32_t poff = nvalid ? (uint32_t)(nrow * (K / 2) + 16 * h) : kOOB;
  const uint32_t coff = nvalid ? (uint32_t)(nrow * nkb) : kOOB;

  // One resource per array for the whole kernel; kb is wave-uniform and
  // moves the loads through the scalar offset field.  Eight buffer loads go
  // straight into LDS buffer `buf`.
  const __amdgpu_buffer_rsrc_t rx = rsrc_whole(g.X, xbytes);
  const __amdgpu_buffer_rsrc_t rp = rsrc_whole(W.packed, pbytes);
  const __amdgpu_buffer_rsrc_t rc = rsrc_whole(W.codes, cbytes);
  const __amdgpu_buffer_rsrc_t rsc = rsrc_whole(W.scales, sbytes);
  // X load j (0..7) of step kb fills rows 64 w + 8 j .. +7 of buffer `buf`;
  // weight load j (0..2) brings the packed bytes, the code, the scale.
  auto load_xj = [&](int j, uint16_t* buf, int kb) {
    const uint32_t k = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rx, (__attribute__((address_space(3))) void*)(buf + (64 * wave + 8 * j) * kXRow), 16,
        xoff[j], k * (kBlock * 2), 0, 0);
  };
  auto load_p = [&](WRegs& R, int kb) {
    const uint32_t k = (uint32_t)__builtin_amdgcn_readfirstlane(kb);
    R.p = bload128s(rp, poff, k * (kBlock / 2));
  };
  // The 8-bit codes of blocks kb4 .. kb4+3 of the lane's row (kb4 a multiple
  // of 4 and K / 64 too, so the 4 bytes are aligned) and their second-level
  // scale (a group of 256 blocks starts at a multiple of 4, so the four
  // blocks share it): one load of each per four steps.
  uint32_t crun_cur = 0, crun_next = 0;
  float srun_cur = 0.0f, srun_next = 0.0f;
  auto load_run_j = [&](int j, int kb4) {
    const uint32_t k = (uint32_t)__builtin_amdgcn_readfirstlane(kb4);
    if (j == 0)
      crun_next = bload32s(rc, coff, k);
    else
      srun_next = __uint_as_float(bload32(rsc, coff == kOOB ? kOOB : ((coff + k) / kDQBlock) * 4u));
  };
  auto load_x = [&](uint16_t* buf, int kb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) load_xj(j, buf, kb);
  };
  auto word = [](const FwdWRegs& R, int t) -> uint32_t {
    return t == 0 ? R.p.x : t == 1 ? R.p.y : t == 2 ? R.p.z : R.p.w;
  };
  // Operand of MFMA step t for token tile i: X row 32 i + c, k = 32 h + 8 t.
  auto xfrag = [&](const uint16_t* buf, int i, int t) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(buf + 32 * i * kXRow + xrd[t]);
  };
  // The levels of byte e of a packed word (high nibble, low nibble): one
  // 8-byte read of the pair table at the byte times 8.
  const char* q44b = reinterpret_cast<const char*>(q44);
  auto levels = [&](uint32_t w, int e) -> float2 {
    return *reinterpret_cast<const float2*>(q44b + (__builtin_amdgcn_ubfe(w, 8 * e, 8) << 3));
  };
  auto decode_all = [&](const FwdWRegs& R, FwdBFrag& F, uint32_t code, float sc) {
    const float ah = absmax_decode_tab((int)code, sc, mean, q8);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 lv = levels(word(R, t), e);
        F.d[t][e] = pack_bf16x2(lv.x * ah, lv.y * ah);
      }
  };

  f32x16_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // Register sets: W(j) in wr[j % 4] from its load (step j-3) to its decode
  // (step j-1); the decoded W(j) in bf[j % 2] during step j.  X(j) is in LDS
  // buffer j % 4 from its load (step j-3) to step j.
  WRegs wr[4];
  FwdBFrag bf[2];
  bf16x8_t a[2][8];
  __syncthreads();   // tables
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    load_x(xbuf[j], min(kz0 + j, kz1 - 1));
    load_p(wr[j], min(kz0 + j, kz1 - 1));
    if (j == 0) {
      load_run_j(0, kz0);
      load_run_j(1, kz0);
    }
  }
  crun_cur = crun_next;
  srun_cur = srun_next;
  // The loads of steps 0 and 1 must have arrived (step 2's may still be in
  // flight) before the barrier publishes X(0) and X(1): the last slots of
  // step 0 read the first operands of step 1, which other waves loaded.
  decode_all(wr[0], bf[0], crun_cur & 0xffu, srun_cur);
  __builtin_amdgcn_s_waitcnt(wait_vm(kLoads, 0));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 8; ++i) a[0][i] = xfrag(xbuf[0], i, 0);

  // One K-step; P = kb % kFwdUnroll selects the register sets.
  auto step = [&](auto Pc, int kb) {
    constexpr int P = decltype(Pc)::value;
    const WRegs& wdec = wr[(P + 1) % 4];
    WRegs& wload = wr[(P + 3) % 4];
    const FwdBFrag& bc = bf[P % 2];
    FwdBFrag& bn = bf[(P + 1) % 2];
    // kb % 4 == P: the loop starts at 0 and steps by 4
    const uint16_t* xcur = xbuf[P];
    const uint16_t* xnext = xbuf[(P + 1) % kXBufs];
    // Block kb+1 is decoded here: byte (kb+1) % 4 of its run, which is the
    // next run at P == 3.
    const uint32_t dcode = ((P == 3 ? crun_next : crun_cur) >> (8 * ((P + 1) % 4))) & 0xffu;
    const float dsc = P == 3 ? srun_next : srun_cur;
    // Run loads at P == 1: blocks kb+3 .. kb+6 (kb+3 is a multiple of 4), or
    // the last run once those are past the end.
    constexpr int kStepLoads = kLoads + (P == 1 ? kRunLoads : 0);
    const int krun = min(kb + 3, kz1 - 4);

    // 8 X loads into the buffer of step kb-1 (its operand reads by this
    // wave completed before the last barrier), then the weight loads.  This
    // step's 9 loads (11 at P == 1; for step kb+3) go out one per MFMA slot,
    // so that the workgroup's waves, released together by the barrier, do
    // not queue all their loads at the address unit before their first MFMA.
    const int kload = min(kb + 3, kz1 - 1);
    uint16_t* const xload = xbuf[(P + 3) % kXBufs];
    const float q8v = q8[dcode];
    float ah = 0.0f;
    float lh[16], ll[16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int t = u / 8, i = u % 8;
      acc[i] = mfma_32x32x16(as_frag(bc.d[t]), a[t & 1][i], acc[i]);
      if (u < 8) load_xj(u, xload, kload);
      else if (u == 8) load_p(wload, kload);
      else if (P == 1 && u < 9 + kRunLoads) load_run_j(u - 9, krun);
      if (t < 3) a[(t + 1) & 1][i] = xfrag(xcur, i, t + 1);
      else a[0][i] = xfrag(xnext, i, 0);
      {
        if (u < 16) {
          // both levels of byte u % 4 of word u / 4 in one read
          const float2 lv = levels(word(wdec, u / 4), u % 4);
          lh[u] = lv.x;
          ll[u] = lv.y;
        }
        if (u == 2) {
#pragma clang fp contract(off)
          const float p = q8v * dsc;
          ah = p + mean;
        }
        if (u >= 16) {
          const int v = u - 16;
          bn.d[v / 4][v % 4] = pack_bf16x2(lh[v] * ah, ll[v] * ah);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // X(kb+2) (loaded during step kb-1) must be in LDS, from every wave,
    // before step kb+1 reads it: wait until at most this step's loads are
    // outstanding, then barrier.
    __builtin_amdgcn_s_waitcnt(wait_vm(kStepLoads, 0xF));
    __builtin_amdgcn_s_barrier();
    if constexpr (P == 3) {
      crun_cur = crun_next;
      srun_cur = srun_next;
    }
  };
  for (int kb = kz0; kb < kz1; kb += kFwdUnroll) {
    step(std::integral_constant<int, 0>(), kb);
    step(std::integral_constant<int, 1>(), kb + 1);
    step(std::integral_constant<int, 2>(), kb + 2);
    step(std::integral_constant<int, 3>(), kb + 3);
  }
  __builtin_amdgcn_s_waitcnt(0);   // no load into LDS outlives the loop

  // Adapter term: acc += (s B) T^T over r in steps of 16 (natural order).
  const uint16_t* const Tp = upw ? g.T2 : g.T;
  const uint16_t* const Bp = upw ? g.B2 : g.B;
  const int r = upw ? g.r2 : g.r;
  const float sc = upw ? g.s2 : g.s;
  const int radd = zsplit == 0 ? r : 0;   // the adapter term goes into split 0 only
  for (int r0 = 0; r0 < radd; r0 += 16) {
    const int rr = r0 + 8 * h;
    uint4 bv = make_uint4(0, 0, 0, 0);
    if (nvalid && rr < r) {
      bv = *reinterpret_cast<const uint4*>(Bp + nrow * r + rr);
      uint32_t wv[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        wv[q] = pack_bf16x2(bf16_to_f32(wv[q] & 0xffffu) * sc, bf16_to_f32(wv[q] >> 16) * sc);
      bv = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, bv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + 32 * i + c;
      uint4 tv = make_uint4(0, 0, 0, 0);
      if (m < g.M && rr < r) tv = *reinterpret_cast<const uint4*>(Tp + (int64_t)m * r + rr);
      acc[i] = mfma_32x32x16(bfr, __builtin_bit_cast(bf16x8_t, tv), acc[i]);
    }
  }

  // Accumulator i: lane holds token m = m0 + 32 i + c and weight rows
  // 8 (v / 4) + 4 h + (v % 4) of the wave's 32; four consecutive rows are
  // one 8-byte piece of Y.
  if (g.part != nullptr) {
    // split contraction: this split's fp32 partial, four features per store
    float* const pz = g.part + (int64_t)zsplit * g.M * N;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + 32 * i + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = nw0 + 8 * q + 4 * h;
        if (m >= g.M || n >= N) continue;   // N % 8 == 0: a group of four is all in or all out
        *reinterpret_cast<float4*>(pz + (int64_t)m * N + n) =
            make_float4(acc[i][4 * q + 0], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
      }
    }
    return;
  }
  uint16_t* const Yp = upw ? g.Y2 : g.Y;
  uint32_t ob[8][4][2];   // the bf16 results, kept for the gated epilogue
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ob[i][q][0] = pack_bf16x2(acc[i][4 * q + 0], acc[i][4 * q + 1]);
      ob[i][q][1] = pack_bf16x2(acc[i][4 * q + 2], acc[i][4 * q + 3]);
    }
  if constexpr (!GATED) {
    // The tile goes out through LDS (the X buffers are free now): rows of
    // 128 weight rows x 2 bytes, tokens 0..127 in xs0 and 128..255 in xs1,
    // the 16-byte pieces of row t XOR-swizzled by t & 15 (conflict-free
    // writes of the lanes' 8-byte pieces and reads of whole rows); then each
    // thread stores 16-byte pieces, a wave four whole 256-byte row segments
    // per store instruction.
    __syncthreads();   // every wave's loads into the X buffers have landed
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* const st = i < 4 ? xs0 : xs1;
      const int row = 32 * (i & 3) + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int piece = (4 * wave + q) ^ (row & 15);
        *reinterpret_cast<uint2*>(st + row * kFwdBN + piece * 8 + 4 * h) =
            make_uint2(ob[i][q][0], ob[i][q][1]);
      }
    }
    __syncthreads();
    const int64_t n0 = (int64_t)tn * kFwdBN;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int gidx = 256 * j + tid;          // 16-byte piece of the tile
      const int row = gidx >> 4, piece = gidx & 15;
      const uint16_t* ld = (row < 128 ? xs0 : xs1) + (row & 127) * kFwdBN;
      const uint4 v = *reinterpret_cast<const uint4*>(ld + ((piece ^ (row & 15)) * 8));
      const int m = m0 + row;
      const int64_t n = n0 + 8 * piece;
      if (m < g.M && n < N)   // N % 8 == 0: a piece is all in or all out
        *reinterpret_cast<uint4*>(Yp + (int64_t)m * N + n) = v;
    }
  } else {
    // Gated: G (waves 0-1) and U (waves 2-3) go through LDS, each as 256
    // token rows of 64 features x 2 bytes (G in xs0, U in xs1), the 16-byte
    // pieces of row t XOR-swizzled by t & 7; then each thread takes matching
    // 16-byte pieces of G and U, forms H = silu(G) U (the elementwise
    // kernel's arithmetic on the same bf16 values) and stores all three, a
    // wave eight whole 128-byte row segments of each per instruction.
    __syncthreads();   // every wave's loads into the X buffers have landed
    {
      uint16_t* const st = upw ? xs1 : xs0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 32 * i + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int piece = (4 * (wave & 1) + q) ^ (row & 7);
          *reinterpret_cast<uint2*>(st + row * (kFwdBN / 2) + piece * 8 + 4 * h) =
              make_uint2(ob[i][q][0], ob[i][q][1]);
        }
      }
    }
    __syncthreads();
    const int64_t n0 = (int64_t)tn * (kFwdBN / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int gidx = 256 * j + tid;          // 16-byte piece of the 256 x 64 tile
      const int row = gidx >> 3, piece = gidx & 7;
      const int off = row * (kFwdBN / 2) + ((piece ^ (row & 7)) * 8);
      const uint4 gv = *reinterpret_cast<const uint4*>(xs0 + off);
      const uint4 uv = *reinterpret_cast<const uint4*>(xs1 + off);
      const int m = m0 + row;
      const int64_t n = n0 + 8 * piece;
      if (m >= g.M || n >= N) continue;   // N % 8 == 0: a piece is all in or all out
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
      uint32_t hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hv[e] = pack_bf16x2(silu_mul_f32(bf16_to_f32(gw[e] & 0xffffu), bf16_to_f32(uw[e] & 0xffffu)),
                            silu_mul_f32(bf16_to_f32(gw[e] >> 16), bf16_to_f32(uw[e] >> 16)));
      const int64_t o = (int64_t)m * N + n;
      *reinterpret_cast<uint4*>(g.Y + o) = gv;
      *reinterpret_cast<uint4*>(g.Y2 + o) = uv;
      *reinterpret_cast<uint4*>(g.H + o) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
    }
  }
}

bool fwd_nf4_supported(int64_t K) { return (K / kBlock) % kFwdUnroll == 0; }

// out = bf16(sum of the split partials (+ out's bf16 values when
// accumulating)), added in the order z = 0, 1, ..., then the old value; one
// thread per 8 consecutive outputs (n8 = stride / 8).
__global__ void __launch_bounds__(256)
k_split_reduce(const float* __restrict__ part, int splits, int64_t stride, int64_t n8,
               uint16_t* __restrict__ out, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int z = 0; z < splits; ++z) {
    const float4* p = reinterpret_cast<const float4*>(part + (int64_t)z * stride) + 2 * i;
    const float4 a = p[0], b = p[1];
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  uint4* const o = reinterpret_cast<uint4*>(out) + i;
  if (accumulate) {
    const uint4 old = *o;
    const uint32_t ow[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] += bf16_to_f32(ow[e] & 0xffffu);
      v[2 * e + 1] += bf16_to_f32(ow[e] >> 16);
    }
  }
  *o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7]));
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t stride, uint16_t* out,
                               bool accumulate, hipStream_t st, hipEvent_t stop) {
  const int64_t n8 = stride / 8;
  hipExtLaunchKernelGGL(k_split_reduce, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                        nullptr, stop, 0, part, splits, stride, n8, out, accumulate ? 1 : 0);
  return hipGetLastError();
}

int fwd_split_len(int64_t M, int64_t K, int64_t N) {
  const int64_t nk = K / kBlock;
  const int64_t tiles = ((M + kFwdBM - 1) / kFwdBM) * ((N + kFwdBN - 1) / kFwdBN);
  if (tiles >= 128 || nk < 2 * kFwdUnroll) return 0;   // two splits do not pay for the partials
  int64_t splits = 256 / tiles;
  if (splits > nk / kFwdUnroll) splits = nk / kFwdUnroll;
  if (splits < 2) return 0;
  const int64_t per = (nk + splits - 1) / splits;
  return (int)(((per + kFwdUnroll - 1) / kFwdUnroll) * kFwdUnroll);
}

hipError_t launch_fwd_gated(const uint16_t* X, int64_t M, const NF4Weight& wg, const uint16_t* Tg,
                            const uint16_t* Bg, int rg, float sg, const NF4Weight& wu,
                            const uint16_t* Tu, const uint16_t* Bu, int ru, float su, uint16_t* G,
                            uint16_t* U, uint16_t* H, hipStream_t st) {
  if (!fwd_nf4_supported(wg.K) || wg.K != wu.K || wg.N != wu.N || wg.bf16 || wu.bf16)
    return hipErrorInvalidValue;
  FwdArgs g{};
  g.X = X; g.M = (int)M; g.w = wg; g.T = Tg; g.B = Bg; g.r = rg; g.s = sg; g.Y = G;
  g.w2 = wu; g.T2 = Tu; g.B2 = Bu; g.r2 = ru; g.s2 = su; g.Y2 = U; g.H = H;
  g.tiles_m = (int)((M + kFwdBM - 1) / kFwdBM);
  g.tiles_n = (int)((wg.N + kFwdBN / 2 - 1) / (kFwdBN / 2));
  g.group_m = group_for(g.tiles_m, g.tiles_n, (double)kFwdBM * wg.K * 2,
                        (double)kFwdBN * wg.K * 0.52);
  hipLaunchKernelGGL(k_fwd_nf4<true>, dim3(g.tiles_m * g.tiles_n), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_fwd_nf4(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* T,
                          const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st,
                          float* part, int kz_len, Span sp, int tn_base) {
  if (!fwd_nf4_supported(w.K) || w.bf16) return hipErrorInvalidValue;
  FwdArgs g{};
  g.X = X; g.M = (int)M; g.w = w; g.T = T; g.B = B; g.r = r; g.s = s; g.Y = Y;
  g.tiles_m = (int)((M + kFwdBM - 1) / kFwdBM);
  g.tiles_n = (int)((w.N + kFwdBN - 1) / kFwdBN) - tn_base;
  g.tn_base = tn_base;
  if (tn_base < 0 || g.tiles_n < 1 || (tn_base > 0 && part != nullptr)) return hipErrorInvalidValue;
  g.group_m = group_for(g.tiles_m, g.tiles_n, (double)kFwdBM * w.K * 2,
                        (double)kFwdBN * w.K * 0.52);
  const int64_t nk = w.K / kBlock;
  const int splits = (part != nullptr && kz_len > 0) ? (int)((nk + kz_len - 1) / kz_len) : 1;
  if (splits > 1) {
    g.part = part;
    g.kz_len = kz_len;
  }
  hipExtLaunchKernelGGL(k_fwd_nf4<false>, dim3(g.tiles_m * g.tiles_n * splits), dim3(256), 0, st,
                        sp.start, splits > 1 ? nullptr : sp.stop, 0, g);
  if (splits > 1) return launch_split_reduce(part, splits, M * w.N, Y, false, st, sp.stop);
  return hipGetLastError();
}

}  // namespace qlk
