// Device-side helpers shared by the gfx950 kernels of the QLoRA NF4 library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace qlk {

// The 16 NF4 levels as fp32 bit patterns, ascending.  They are the standard
// normal quantiles that give every bin the same probability mass (8 on the
// positive side, 7 on the negative side, plus an exact zero), divided by the
// outermost quantile so that the range is exactly [-1, 1]; the outermost
// probability is 1 - (1/30 + 1/32)/2.  (auryth.ai "QLoRA", NF4 box;
// llm-compass "QLoRA", 方法与公式 item 1.)  Each value was evaluated in high
// precision and rounded once to fp32.
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu,
    0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
    0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

constexpr int kBlock = 64;      // weights per absmax constant
constexpr int kDQBlock = 256;   // constants per second-level scale

__device__ __forceinline__ float nf4_level(int i) { return __uint_as_float(kNF4Bits[i]); }

// 8-bit level i of the symmetric linear code: the correctly rounded fp32
// quotient (i - 127) / 127.  Computed as a multiply by fl(1/127) followed by
// one fused correction step, q = fma(fma(-q0, 127, x), fl(1/127), q0) with
// q0 = x fl(1/127); for the 256 numerators x = -127 .. 128 this equals the
// correctly rounded quotient (verified exhaustively in exact rational
// arithmetic), in three instructions instead of a division.
__device__ __forceinline__ float dq_level(int i) {
#pragma clang fp contract(off)
  const float x = (float)(i - 127);
  const float inv = 1.0f / 127.0f;
  const float q0 = x * inv;
  const float r = __builtin_fmaf(-q0, 127.0f, x);
  return __builtin_fmaf(r, inv, q0);
}

// Decision threshold between 8-bit levels i and i+1: their exact midpoint
// (exact in fp64) rounded toward -inf, so that for any fp32 n
// "n > threshold" <=> "n is strictly above the midpoint".  Ties (n equal to
// a representable midpoint) therefore go to the lower index.  The 4-bit
// codebooks carry thresholds built the same way (Codebook4).
__device__ __forceinline__ float dq_threshold(int i) {
  double m = ((double)dq_level(i) + (double)dq_level(i + 1)) * 0.5;
  return __double2float_rd(m);
}

// SiLU gating of the MLP glue: silu(g) u = g sigmoid(g) u, evaluated left
// to right in fp32 (shared by the elementwise kernel and the fused gate/up
// forward, which therefore give the same bits).
__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_mul_f32(float g, float u) { return g * sigmoidf_(g) * u; }

// a_hat = fp32(fp32(Q8[code] * scale) + mean): two separately rounded ops.
__device__ __forceinline__ float absmax_decode(int code, float scale, float mean) {
#pragma clang fp contract(off)
  float q = dq_level(code);
  float p = q * scale;
  return p + mean;
}

// Same decode with the 8-bit levels read from a table (e.g. in LDS) that
// holds dq_level(i) at index i.
__device__ __forceinline__ float absmax_decode_tab(int code, float scale, float mean,
                                                   const float* q8) {
#pragma clang fp contract(off)
  float p = q8[code] * scale;
  return p + mean;
}

// Decode context handed to the NF4 tile loaders: the 16 NF4 levels and the
// 256 8-bit levels (both in LDS) and the tensor's mean constant.
struct Dec {
  const float* q4;
  const float* q8;
  float mean;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round two fp32 values to bf16 (round-to-nearest-even, hardware convert) and
// pack them, `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Select two 16-bit halves: result = (lo half of x, lo half of y) or the
// high halves, via the byte permute unit.
__device__ __forceinline__ uint32_t lo16x2(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// Transpose an 8x8 tile of 16-bit values held as 8 rows of 4 packed words:
// in[i].w[j] = (e[i][2j], e[i][2j+1]);  out[j].w[k] = (e[2k][j], e[2k+1][j]).
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = reinterpret_cast<const uint32_t*>(&in[i]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t x = r[2 * k][j >> 1], y = r[2 * k + 1][j >> 1];
      w[k] = (j & 1) ? hi16x2(x, y) : lo16x2(x, y);
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;

// LDS transpose read of 16-bit elements (gfx950 ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane t receives element (t % 4) of the 8-byte pieces
// that source lanes 4s + t/4 point at, for s = 0..3.  If source lane 4s + u of
// a group points at row r0 + s, column c0 + 4u of a row-major tile, lane t
// receives column c0 + t of rows r0 .. r0+3.
__device__ __forceinline__ v4s_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p));
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// ----------------------------- buffer loads ---------------------------------
//
// Loads go through raw buffer resources.  Each loader fixes its per-lane byte
// offsets once per phase (init); every K-step only moves the resource base by
// a scalar amount, so the loads cost no vector address arithmetic.  A lane
// whose element lies outside the operand uses an offset past the end of the
// buffer and the hardware returns zero.

constexpr uint32_t kOOB = 0x80000000u;       // offset beyond any accepted buffer
constexpr int kRsrcWord3 = 0x00020000;        // raw buffer, 32-bit data format

// A resource over a whole array, built once per kernel.  Loads then add a
// wave-uniform byte offset in the instruction's scalar offset field, so a
// K-step costs one scalar add instead of a new resource.  Out-of-range lanes
// still use kOOB in the per-lane offset; every in-range access lies inside
// the array, so the result does not depend on whether the hardware's range
// check includes the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_whole(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint2 bload64s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t bload32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t bload8s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
}


// ------------------------- workgroup -> tile order ---------------------------

constexpr int kXCDs = 8;   // the hardware deals workgroup ids round-robin over 8 XCDs
constexpr int kCUs = 256;  // compute units: one round of one-workgroup-per-CU tiles

// Tile coordinates of workgroup `bid`: ids are first regrouped so that the
// workgroups one XCD receives (bid = x, x+8, x+16, ...) get consecutive
// positions, then walked in groups of `group_p` tile rows across all tile
// columns.  Both steps are bijections on [0, tiles).
__device__ __forceinline__ void tile_coords(int bid, int tiles_p, int tiles_q, int group_p, int& tp,
                                            int& tq) {
  const int total = tiles_p * tiles_q;
  const int full = (total / kXCDs) * kXCDs;
  int t = bid;
  if (bid < full) t = (bid % kXCDs) * (full / kXCDs) + bid / kXCDs;
  const int per_group = group_p * tiles_q;
  const int gi = t / per_group;
  const int first = gi * group_p;
  const int gp = min(group_p, tiles_p - first);
  const int rem = t - gi * per_group;
  tp = first + rem % gp;
  tq = rem / gp;
}

}  // namespace qlk
