// C ABI of the QLoRA NF4 library: argument validation and dispatch.
// Every check runs on the host before anything is enqueued, so a non-zero
// status always means that no kernel was launched.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/qlora.h"
#include "kernels.h"

namespace {

constexpr int kBlock = 64;
constexpr int kDQBlock = 256;
constexpr int64_t kMaxDim = (int64_t)1 << 30;   // keeps every tile index in int
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;

constexpr int kMaxRank = 256;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The kernels read adapter rows (A, B, T, U) as 16-byte pieces, so they take
// a rank that is a multiple of 8.  Any other rank r is run as the next
// multiple of 8, rp, on zero-padded copies of A (extra zero rows) and B
// (extra zero columns) in the workspace; the padded T, U, dA and dB then hold
// zeros in the extra rows or columns, every product the caller sees is the
// same sum (plus exact zero terms), and T, dA and dB are cut back to r
// columns or rows.  s stays alpha / r.
inline int padded_rank(int r) { return (r + 7) & ~7; }
struct PadPlan {
  int rp;
  size_t off_A, off_B, off_T, off_dA, off_dB, bytes;
};
// `base` is the kernels' own workspace need for rank rp; the padded copies
// follow it.
PadPlan plan_pad(size_t base, int64_t M, int64_t K, int64_t N, int r, bool bwd) {
  PadPlan p{};
  p.rp = padded_rank(r);
  size_t off = align256(base);
  if (p.rp != r) {
    const size_t rp = (size_t)p.rp;
    p.off_A = off; off += align256(rp * K * 2);
    p.off_B = off; off += align256((size_t)N * rp * 2);
    p.off_T = off; off += align256((size_t)M * rp * 2);
    if (bwd) {
      p.off_dA = off; off += align256(rp * K * 4);
      p.off_dB = off; off += align256((size_t)N * rp * 4);
    }
    p.bytes = off;
  } else {
    p.bytes = base;
  }
  return p;
}
PadPlan fwd_layout(int64_t M, int64_t K, int64_t N, int r, bool nf4) {
  return plan_pad(qlk::plan_fwd(M, K, N, padded_rank(r), nf4).bytes, M, K, N, r, false);
}
PadPlan bwd_layout(int64_t M, int64_t K, int64_t N, int r, bool dx) {
  return plan_pad(qlk::plan_bwd(M, K, N, padded_rank(r), dx).bytes, M, K, N, r, true);
}
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int launch_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

// NF4 level bit patterns (the same values the kernels embed; see
// device_common.h for their definition).
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu,
    0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
    0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

int check_weight_shape(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % kBlock != 0) return QLORA_ERR_SHAPE;
  if (N > kMaxDim || K > kMaxDim) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

// Checks shared by both weight formats; `weight_bytes` is the size of the
// stored base weight the kernels address with buffer offsets.
int check_linear_common(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* A,
                        const uint16_t* B, int r, float alpha, bool weight_null, int64_t weight_bytes) {
  if (!X || !A || !B || weight_null) return QLORA_ERR_NULL;
  if (M <= 0 || M > kMaxDim) return QLORA_ERR_SHAPE;
  int st = check_weight_shape(N, K);
  if (st) return st;
  if (N % 8 != 0) return QLORA_ERR_SHAPE;
  if (r < 1 || r > kMaxRank) return QLORA_ERR_SHAPE;
  // The kernels address X, dY, Y, dX and the stored weight with 32-bit
  // buffer offsets and mark out-of-range lanes with offset 2^31.
  if (M * K * 2 >= kMaxBufferBytes || M * N * 2 >= kMaxBufferBytes || weight_bytes >= kMaxBufferBytes)
    return QLORA_ERR_SHAPE;
  if (!isfinite(alpha)) return QLORA_ERR_ARG;
  if (!aligned16(X) || !aligned16(A) || !aligned16(B)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_linear(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                 const uint8_t* codes, const float* scales, const float* mean, const uint16_t* A,
                 const uint16_t* B, int r, float alpha) {
  const bool wnull = !packed || !codes || !scales || !mean;
  int st = check_linear_common(X, M, K, N, A, B, r, alpha, wnull, wnull ? 0 : N * K / 2);
  if (st) return st;
  if (!aligned16(packed) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_linear_bf16(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                      const uint16_t* A, const uint16_t* B, int r, float alpha) {
  int st = check_linear_common(X, M, K, N, A, B, r, alpha, !W, W ? N * K * 2 : 0);
  if (st) return st;
  return aligned16(W) ? QLORA_OK : QLORA_ERR_ALIGN;
}

qlk::NF4Weight weight(const uint8_t* packed, const uint8_t* codes, const float* scales,
                      const float* mean, int64_t N, int64_t K) {
  qlk::NF4Weight w;
  w.packed = packed; w.codes = codes; w.scales = scales; w.mean = mean; w.N = N; w.K = K;
  return w;
}

qlk::NF4Weight weight_bf16(const uint16_t* W, int64_t N, int64_t K) {
  qlk::NF4Weight w;
  w.packed = nullptr; w.codes = nullptr; w.scales = nullptr; w.mean = nullptr;
  w.N = N; w.K = K; w.bf16 = W;
  return w;
}

int fwd_common(const uint16_t* X, int64_t M, int64_t K, int64_t N, const qlk::NF4Weight& w,
               const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* Y,
               uint16_t* T_out, void* workspace, size_t workspace_bytes, void* stream,
               const uint16_t* Xa = nullptr, const qlk::Timing* tm = nullptr) {
  if (!Y) return QLORA_ERR_NULL;
  if (!aligned16(Y) || (T_out && !aligned16(T_out))) return QLORA_ERR_ALIGN;
  const int rp = padded_rank(r);
  const qlk::FwdPlan plan = qlk::plan_fwd(M, K, N, rp, w.bf16 == nullptr);
  const PadPlan pad = plan_pad(plan.bytes, M, K, N, r, false);
  if (workspace_bytes < pad.bytes || (pad.bytes && !workspace)) return QLORA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return QLORA_ERR_ALIGN;
  const float s = alpha / (float)r;
  const hipStream_t st = as_stream(stream);
  if (rp == r)
    return launch_status(qlk::launch_qlora_fwd(X, M, w, A, B, r, s, Y, T_out, workspace, plan, st,
                                               Xa, tm));
  char* base = reinterpret_cast<char*>(workspace);
  uint16_t* Ap = reinterpret_cast<uint16_t*>(base + pad.off_A);
  uint16_t* Bp = reinterpret_cast<uint16_t*>(base + pad.off_B);
  uint16_t* Tp = reinterpret_cast<uint16_t*>(base + pad.off_T);
  hipError_t e = qlk::launch_pad2d(A, r, K, Ap, rp, K, st);
  if (e == hipSuccess) e = qlk::launch_pad2d(B, N, r, Bp, N, rp, st);
  if (e == hipSuccess) e = qlk::launch_qlora_fwd(X, M, w, Ap, Bp, rp, s, Y, Tp, workspace, plan, st, Xa, tm);
  if (e == hipSuccess && T_out) e = qlk::launch_pad2d(Tp, M, rp, T_out, M, r, st);
  return launch_status(e);
}

// The backward's own arguments (beyond those check_linear covers).
int check_bwd_args(const uint16_t* dY, const uint16_t* T, const uint16_t* dX, const float* dA,
                   const float* dB, int flags) {
  if (!dY || !dA || !dB) return QLORA_ERR_NULL;
  if (flags & ~QLORA_BWD_ACCUMULATE_DX) return QLORA_ERR_ARG;
  if (!aligned16(dY) || !aligned16(dA) || !aligned16(dB) || (dX && !aligned16(dX)) ||
      (T && !aligned16(T)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int bwd_common(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K, int64_t N,
               const qlk::NF4Weight& w, const uint16_t* A, const uint16_t* B, int r, float alpha,
               const uint16_t* T, uint16_t* dX, float* dA, float* dB, int flags, void* workspace,
               size_t workspace_bytes, void* stream, const uint32_t* mask = nullptr,
               float keep_scale = 1.0f, const qlk::Timing* tm = nullptr) {
  const int bad = check_bwd_args(dY, T, dX, dA, dB, flags);
  if (bad) return bad;
  const int rp = padded_rank(r);
  const qlk::BwdPlan plan = qlk::plan_bwd(M, K, N, rp, dX != nullptr);
  const PadPlan pad = plan_pad(plan.bytes, M, K, N, r, true);
  if (workspace_bytes < pad.bytes || !workspace) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;
  const float s = alpha / (float)r;
  const bool acc = (flags & QLORA_BWD_ACCUMULATE_DX) != 0;
  const hipStream_t st = as_stream(stream);
  if (rp == r)
    return launch_status(qlk::launch_qlora_bwd(dY, X, M, w, A, B, r, s, T, dX, dA, dB, acc,
                                               workspace, plan, st, mask, keep_scale, tm));
  char* base = reinterpret_cast<char*>(workspace);
  uint16_t* Ap = reinterpret_cast<uint16_t*>(base + pad.off_A);
  uint16_t* Bp = reinterpret_cast<uint16_t*>(base + pad.off_B);
  uint16_t* Tp = reinterpret_cast<uint16_t*>(base + pad.off_T);
  float* dAp = reinterpret_cast<float*>(base + pad.off_dA);
  float* dBp = reinterpret_cast<float*>(base + pad.off_dB);
  hipError_t e = qlk::launch_pad2d(A, r, K, Ap, rp, K, st);
  if (e == hipSuccess) e = qlk::launch_pad2d(B, N, r, Bp, N, rp, st);
  if (e == hipSuccess && T) e = qlk::launch_pad2d(T, M, r, Tp, M, rp, st);
  if (e == hipSuccess)
    e = qlk::launch_qlora_bwd(dY, X, M, w, Ap, Bp, rp, s, T ? Tp : nullptr, dX, dAp, dBp, acc,
                              workspace, plan, st, mask, keep_scale, tm);
  if (e == hipSuccess) e = qlk::launch_pad2d(dAp, rp, K, dA, r, K, st);
  if (e == hipSuccess) e = qlk::launch_pad2d(dBp, N, rp, dB, N, r, st);
  return launch_status(e);
}

int check_codebook(const float* levels) {
  if (!levels) return QLORA_ERR_NULL;
  for (int i = 0; i < 16; ++i)
    if (!isfinite(levels[i]) || (i > 0 && !(levels[i - 1] < levels[i]))) return QLORA_ERR_ARG;
  return QLORA_OK;
}

// The caller's events (hipEvent_t as void*) in the launchers' form; null for
// an untimed call.
const qlk::Timing* to_timing(const qlora_timing* t, qlk::Timing& out) {
  if (!t) return nullptr;
  static_assert(QLORA_KERNEL_COUNT == qlk::TK_COUNT, "one event slot per timed kernel");
  for (int k = 0; k < qlk::TK_COUNT; ++k) {
    out.start[k] = reinterpret_cast<hipEvent_t>(t->start[k]);
    out.stop[k] = reinterpret_cast<hipEvent_t>(t->stop[k]);
  }
  return &out;
}

// A second-level table from the caller: 2..256 finite, strictly ascending
// levels (HOST memory).
int check_table8(const float* levels, int n) {
  if (!levels) return QLORA_ERR_NULL;
  if (n < 2 || n > 256) return QLORA_ERR_ARG;
  for (int i = 0; i < n; ++i)
    if (!isfinite(levels[i]) || (i > 0 && !(levels[i - 1] < levels[i]))) return QLORA_ERR_ARG;
  return QLORA_OK;
}

// The 8-bit-float second-level levels: every finite value of the 8-bit float
// with 4 exponent bits (bias 7) and 3 mantissa bits (the all-ones pattern is
// NaN, there are no infinities), divided by its largest value 448, the fp64
// quotient rounded once to fp32; ascending, 253 levels, zero at index 126.
int float8_levels(float* out) {
  double v[128];
  int n = 0;
  for (int b = 0; b < 127; ++b) {          // the non-negative patterns, ascending
    const int e = (b >> 3) & 15, m = b & 7;
    v[n++] = e == 0 ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  }
  int k = 0;
  for (int i = n - 1; i >= 1; --i) out[k++] = (float)(-v[i] / 448.0);
  for (int i = 0; i < n; ++i) out[k++] = (float)(v[i] / 448.0);
  return k;
}

bool valid_p(double p) { return p >= 0.0 && p < 1.0; }   // false for NaN
uint32_t dropout_threshold(double p) { return (uint32_t)floor(p * 4294967296.0); }
float dropout_scale(double p) { return (float)(1.0 / (1.0 - p)); }

int quantize_common(const float* W0, int64_t N, int64_t K, int blocksize, const qlk::Codebook4& cb,
                    uint8_t* packed, float* absmax, void* stream) {
  if (!W0 || !packed || !absmax) return QLORA_ERR_NULL;
  if (blocksize != kBlock) return QLORA_ERR_UNSUPPORTED;
  int st = check_weight_shape(N, K);
  if (st) return st;
  if (N * K / kBlock > (int64_t)0x7fffffff * 32) return QLORA_ERR_SHAPE;
  if (!aligned16(W0) || !aligned16(packed) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_nf4_quantize(W0, N * K, cb, packed, absmax, as_stream(stream)));
}

int dequant_common(const uint8_t* packed, const uint8_t* codes, const float* scales,
                   const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                   const qlk::Codebook4& cb, uint16_t* W_bf16, void* stream) {
  if (!packed || !codes || !scales || !mean || !W_bf16) return QLORA_ERR_NULL;
  if (blocksize != kBlock || dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  int st = check_weight_shape(N, K);
  if (st) return st;
  if (N * K / 32 / 256 > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean) ||
      !aligned16(W_bf16))
    return QLORA_ERR_ALIGN;
  return launch_status(
      qlk::launch_nf4_dequant(packed, codes, scales, mean, N * K, cb, W_bf16, as_stream(stream)));
}

// ---- static scratch of qlora_linear_bwd_noalloc ---------------------------
//
// Callers that cannot allocate (graph capture, serving loops, harnesses that
// forbid it) get a backward whose scratch memory is this file-scope array:
// every GPU the library runs on holds its own copy from module load until the
// process ends.  On the host, `scratch` is only a stand-in for the symbol;
// the device address of each GPU's copy is looked up once per device (with
// that device current) and kept, and only that address is handed to kernels.
// No kernel of the backward needs its scratch to start at zero (every value
// it reads back was written earlier in the same call), so nothing is cleared.
// Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the scratch array on the GPU of `stream` (or of the
// current device for the null stream).
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return QLORA_ERR_LAUNCH;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return QLORA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_LAUNCH;
  std::call_once(g_scratch_once[dev], [dev, cur] {
    hipError_t e = hipSuccess;
    if (dev != cur) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return QLORA_ERR_LAUNCH;
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" {

int nf4_quantize(const float* W0, int64_t N, int64_t K, int blocksize, uint8_t* packed,
                 float* absmax, void* stream) {
  return quantize_common(W0, N, K, blocksize, qlk::nf4_codebook4(), packed, absmax, stream);
}

int codebook_quantize(const float* W0, int64_t N, int64_t K, int blocksize, const float* levels,
                      uint8_t* packed, float* absmax, void* stream) {
  int st = check_codebook(levels);
  if (st) return st;
  return quantize_common(W0, N, K, blocksize, qlk::make_codebook(levels), packed, absmax, stream);
}

int double_quant(const float* absmax, int64_t nblocks, int dq_blocksize, uint8_t* codes,
                 float* scales, float* mean, void* stream) {
  if (!absmax || !codes || !scales || !mean) return QLORA_ERR_NULL;
  if (dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  if (nblocks <= 0 || (nblocks + kDQBlock - 1) / kDQBlock > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(absmax) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean))
    return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_double_quant(absmax, nblocks, codes, scales, mean,
                                                as_stream(stream)));
}

int double_quant_table(const float* absmax, int64_t nblocks, int dq_blocksize,
                       const float* levels, int nlevels, uint8_t* codes, float* scales, float* mean,
                       void* stream) {
  int st = check_table8(levels, nlevels);
  if (st) return st;
  if (!absmax || !codes || !scales || !mean) return QLORA_ERR_NULL;
  if (dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  if (nblocks <= 0 || (nblocks + kDQBlock - 1) / kDQBlock > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(absmax) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean))
    return QLORA_ERR_ALIGN;
  const qlk::Codebook8 cb8 = qlk::make_codebook8(levels, nlevels);
  return launch_status(qlk::launch_double_quant(absmax, nblocks, codes, scales, mean,
                                                as_stream(stream), &cb8));
}

int absmax_dequant(const uint8_t* codes, const float* scales, const float* mean, int64_t nblocks,
                   int dq_blocksize, const float* levels, int nlevels, float* out, void* stream) {
  int st = check_table8(levels, nlevels);
  if (st) return st;
  if (!codes || !scales || !mean || !out) return QLORA_ERR_NULL;
  if (dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  if (nblocks <= 0 || (nblocks + 255) / 256 > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(mean) || !aligned16(out))
    return QLORA_ERR_ALIGN;
  const qlk::Codebook8 cb8 = qlk::make_codebook8(levels, nlevels);
  return launch_status(qlk::launch_absmax_dequant(codes, scales, mean, nblocks, cb8, out,
                                                  as_stream(stream)));
}

int dequant_tables(const uint8_t* packed, const uint8_t* codes, const float* scales,
                   const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                   const float* levels4, const float* levels8, int nlevels8, uint16_t* W_bf16,
                   void* stream) {
  int st = check_table8(levels8, nlevels8);
  if (st) return st;
  if (levels4) {
    st = check_codebook(levels4);
    if (st) return st;
  }
  if (!packed || !codes || !scales || !mean || !W_bf16) return QLORA_ERR_NULL;
  if (blocksize != kBlock || dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  st = check_weight_shape(N, K);
  if (st) return st;
  if (N * K / 32 / 256 > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean) ||
      !aligned16(W_bf16))
    return QLORA_ERR_ALIGN;
  const qlk::Codebook8 cb8 = qlk::make_codebook8(levels8, nlevels8);
  const qlk::Codebook4 cb4 = levels4 ? qlk::make_codebook(levels4) : qlk::nf4_codebook4();
  return launch_status(qlk::launch_nf4_dequant(packed, codes, scales, mean, N * K, cb4, W_bf16,
                                               as_stream(stream), &cb8));
}

int nf4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                uint16_t* W_bf16, void* stream) {
  return dequant_common(packed, codes, scales, mean, N, K, blocksize, dq_blocksize,
                        qlk::nf4_codebook4(), W_bf16, stream);
}

int codebook_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                     const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                     const float* levels, uint16_t* W_bf16, void* stream) {
  int st = check_codebook(levels);
  if (st) return st;
  return dequant_common(packed, codes, scales, mean, N, K, blocksize, dq_blocksize,
                        qlk::make_codebook(levels), W_bf16, stream);
}

int lora_dropout(const uint16_t* X, int64_t M, int64_t K, double p, uint64_t seed, uint16_t* Xd,
                 uint32_t* mask, void* stream) {
  if (!X || !Xd || !mask) return QLORA_ERR_NULL;
  if (M <= 0 || K <= 0 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return QLORA_ERR_SHAPE;
  if (M * K * 2 >= kMaxBufferBytes) return QLORA_ERR_SHAPE;
  if (!valid_p(p)) return QLORA_ERR_ARG;
  if (!aligned16(X) || !aligned16(Xd) || !aligned16(mask)) return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_lora_dropout(X, M * K, dropout_threshold(p), dropout_scale(p),
                                                seed, Xd, mask, as_stream(stream)));
}

int qlora_merge(const uint8_t* packed, const uint8_t* codes, const float* scales,
                const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* W_merged,
                void* stream) {
  if (!packed || !codes || !scales || !mean || !A || !B || !W_merged) return QLORA_ERR_NULL;
  if (blocksize != kBlock || dq_blocksize != kDQBlock) return QLORA_ERR_UNSUPPORTED;
  int st = check_weight_shape(N, K);
  if (st) return st;
  if (N % 8 != 0 || r < 1 || r > kMaxRank) return QLORA_ERR_SHAPE;
  if (N * K > ((int64_t)1 << 40) || (N + 63) / 64 > 65535) return QLORA_ERR_SHAPE;
  if (!isfinite(alpha)) return QLORA_ERR_ARG;
  if (!aligned16(packed) || !aligned16(codes) || !aligned16(scales) || !aligned16(mean) ||
      !aligned16(A) || !aligned16(B) || !aligned16(W_merged))
    return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_merge(weight(packed, codes, scales, mean, N, K), A, B, r,
                                         alpha / (float)r, W_merged, as_stream(stream)));
}

size_t qlora_workspace_bytes(int64_t M, int64_t K, int64_t N, int r, int is_bwd) {
  if (M <= 0 || M > kMaxDim || check_weight_shape(N, K) || r < 1 || r > kMaxRank) return 0;
  return is_bwd ? bwd_layout(M, K, N, r, true).bytes : fwd_layout(M, K, N, r, true).bytes;
}

int qlora_linear_fwd_timed(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                           const uint8_t* packed, const uint8_t* codes, const float* scales,
                           const float* mean, const uint16_t* A, const uint16_t* B, int r,
                           float alpha, uint16_t* Y, uint16_t* T_out, void* workspace,
                           size_t workspace_bytes, void* stream, const qlora_timing* timing) {
  int st = check_linear(X, M, K, N, packed, codes, scales, mean, A, B, r, alpha);
  if (st) return st;
  qlk::Timing tm;
  const qlk::Timing* tp = to_timing(timing, tm);
  return fwd_common(X, M, K, N, weight(packed, codes, scales, mean, N, K), A, B, r, alpha, Y,
                    T_out, workspace, workspace_bytes, stream, nullptr, tp);
}

int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                     const uint8_t* codes, const float* scales, const float* mean,
                     const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* Y,
                     uint16_t* T_out, void* workspace, size_t workspace_bytes, void* stream) {
  return qlora_linear_fwd_timed(X, M, K, N, packed, codes, scales, mean, A, B, r, alpha, Y, T_out,
                                workspace, workspace_bytes, stream, nullptr);
}

int qlora_linear_fwd_dropout(const uint16_t* X, const uint16_t* Xd, int64_t M, int64_t K,
                             int64_t N, const uint8_t* packed, const uint8_t* codes,
                             const float* scales, const float* mean, const uint16_t* A,
                             const uint16_t* B, int r, float alpha, uint16_t* Y,
                             uint16_t* T_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_linear(X, M, K, N, packed, codes, scales, mean, A, B, r, alpha);
  if (st) return st;
  if (!Xd) return QLORA_ERR_NULL;
  if (!aligned16(Xd)) return QLORA_ERR_ALIGN;
  return fwd_common(X, M, K, N, weight(packed, codes, scales, mean, N, K), A, B, r, alpha, Y,
                    T_out, workspace, workspace_bytes, stream, Xd);
}

int qlora_linear_fwd_bf16(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                          const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* Y,
                          uint16_t* T_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_linear_bf16(X, M, K, N, W, A, B, r, alpha);
  if (st) return st;
  return fwd_common(X, M, K, N, weight_bf16(W, N, K), A, B, r, alpha, Y, T_out, workspace,
                    workspace_bytes, stream);
}

int qlora_linear_bwd_timed(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K,
                           int64_t N, const uint8_t* packed, const uint8_t* codes,
                           const float* scales, const float* mean, const uint16_t* A,
                           const uint16_t* B, int r, float alpha, const uint16_t* T, uint16_t* dX,
                           float* dA, float* dB, int flags, void* workspace,
                           size_t workspace_bytes, void* stream, const qlora_timing* timing) {
  int st = check_linear(X, M, K, N, packed, codes, scales, mean, A, B, r, alpha);
  if (st) return st;
  qlk::Timing tm;
  const qlk::Timing* tp = to_timing(timing, tm);
  return bwd_common(dY, X, M, K, N, weight(packed, codes, scales, mean, N, K), A, B, r, alpha, T,
                    dX, dA, dB, flags, workspace, workspace_bytes, stream, nullptr, 1.0f, tp);
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K, int64_t N,
                     const uint8_t* packed, const uint8_t* codes, const float* scales,
                     const float* mean, const uint16_t* A, const uint16_t* B, int r, float alpha,
                     const uint16_t* T, uint16_t* dX, float* dA, float* dB, int flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return qlora_linear_bwd_timed(dY, X, M, K, N, packed, codes, scales, mean, A, B, r, alpha, T,
                                dX, dA, dB, flags, workspace, workspace_bytes, stream, nullptr);
}

int qlora_linear_bwd_noalloc(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K,
                             int64_t N, const uint8_t* packed, const uint8_t* codes,
                             const float* scales, const float* mean, const uint16_t* A,
                             const uint16_t* B, int r, float alpha, const uint16_t* T, uint16_t* dX,
                             float* dA, float* dB, int flags, void* stream) {
  int st = check_linear(X, M, K, N, packed, codes, scales, mean, A, B, r, alpha);
  if (st) return st;
  st = check_bwd_args(dY, T, dX, dA, dB, flags);
  if (st) return st;
  if (bwd_layout(M, K, N, r, dX != nullptr).bytes > (size_t)QLORA_NOALLOC_SCRATCH_BYTES)
    return QLORA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(as_stream(stream), &ws);
  if (st) return st;
  return bwd_common(dY, X, M, K, N, weight(packed, codes, scales, mean, N, K), A, B, r, alpha, T,
                    dX, dA, dB, flags, ws, (size_t)QLORA_NOALLOC_SCRATCH_BYTES, stream);
}

int qlora_linear_bwd_dropout(const uint16_t* dY, const uint16_t* Xd, const uint32_t* mask,
                             double p, int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                             const uint8_t* codes, const float* scales, const float* mean,
                             const uint16_t* A, const uint16_t* B, int r, float alpha,
                             const uint16_t* T, uint16_t* dX, float* dA, float* dB, int flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
  // Xd takes the place of X: it is the adapter input that feeds T and dA.
  int st = check_linear(Xd, M, K, N, packed, codes, scales, mean, A, B, r, alpha);
  if (st) return st;
  if (!mask) return QLORA_ERR_NULL;
  if (!aligned16(mask)) return QLORA_ERR_ALIGN;
  if (!valid_p(p)) return QLORA_ERR_ARG;
  return bwd_common(dY, Xd, M, K, N, weight(packed, codes, scales, mean, N, K), A, B, r, alpha, T,
                    dX, dA, dB, flags, workspace, workspace_bytes, stream, mask, dropout_scale(p));
}

int qlora_linear_bwd_bf16(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K, int64_t N,
                          const uint16_t* W, const uint16_t* A, const uint16_t* B, int r,
                          float alpha, const uint16_t* T, uint16_t* dX, float* dA, float* dB,
                          int flags, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_linear_bf16(X, M, K, N, W, A, B, r, alpha);
  if (st) return st;
  return bwd_common(dY, X, M, K, N, weight_bf16(W, N, K), A, B, r, alpha, T, dX, dA, dB, flags,
                    workspace, workspace_bytes, stream);
}

int qlora_mlp_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t I,
                  const qlora_lora_linear* gate, const qlora_lora_linear* up, uint16_t* G,
                  uint16_t* U, uint16_t* H, uint16_t* Tg, uint16_t* Tu, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!gate || !up) return QLORA_ERR_NULL;
  const qlora_lora_linear* lin[2] = {gate, up};
  for (const qlora_lora_linear* l : lin) {
    int st = check_linear(X, M, K, I, l->packed, l->codes, l->scales, l->mean, l->A, l->B, l->r,
                          l->alpha);
    if (st) return st;
  }
  if (!G || !U || !H || !Tg || !Tu) return QLORA_ERR_NULL;
  if (!aligned16(G) || !aligned16(U) || !aligned16(H) || !aligned16(Tg) || !aligned16(Tu) ||
      (workspace && !aligned16(workspace)))
    return QLORA_ERR_ALIGN;
  const bool whole_rank = padded_rank(gate->r) == gate->r && padded_rank(up->r) == up->r;
  if (whole_rank && qlk::mlp_fwd_fused(M, K, I)) {
    // One kernel for both projections and the gating; T of each projection
    // goes straight to Tg and Tu, so no workspace is needed.
    qlk::LoraLinear L[2];
    for (int j = 0; j < 2; ++j) {
      const qlora_lora_linear& l = *lin[j];
      L[j].w = weight(l.packed, l.codes, l.scales, l.mean, I, K);
      L[j].A = l.A; L[j].B = l.B; L[j].r = l.r; L[j].s = l.alpha / (float)l.r;
    }
    return launch_status(qlk::launch_mlp_fwd(X, M, L[0], L[1], G, U, H, Tg, Tu, as_stream(stream)));
  }
  // Otherwise the two layer forwards and the elementwise gating, one after
  // the other on the stream (they share the workspace).
  for (const qlora_lora_linear* l : lin) {
    const size_t need = fwd_layout(M, K, I, l->r, true).bytes;
    if (workspace_bytes < need || (need && !workspace)) return QLORA_ERR_WORKSPACE;
  }
  int st = fwd_common(X, M, K, I, weight(gate->packed, gate->codes, gate->scales, gate->mean, I, K),
                      gate->A, gate->B, gate->r, gate->alpha, G, Tg, workspace, workspace_bytes,
                      stream);
  if (st) return st;
  st = fwd_common(X, M, K, I, weight(up->packed, up->codes, up->scales, up->mean, I, K), up->A,
                  up->B, up->r, up->alpha, U, Tu, workspace, workspace_bytes, stream);
  if (st) return st;
  return launch_status(qlk::launch_silu_mul_fwd(G, U, M * I, H, as_stream(stream)));
}

int qlora_mlp_bwd(const uint16_t* dH, const uint16_t* X, int64_t M, int64_t K, int64_t I,
                  const qlora_lora_linear* gate, const qlora_lora_linear* up, const uint16_t* G,
                  const uint16_t* U, const uint16_t* Tg, const uint16_t* Tu, uint16_t* dG,
                  uint16_t* dU, uint16_t* dX, float* dAg, float* dBg, float* dAu, float* dBu,
                  int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!gate || !up) return QLORA_ERR_NULL;
  const qlora_lora_linear* lin[2] = {gate, up};
  for (const qlora_lora_linear* l : lin) {
    int st = check_linear(X, M, K, I, l->packed, l->codes, l->scales, l->mean, l->A, l->B, l->r,
                          l->alpha);
    if (st) return st;
    if (workspace_bytes < bwd_layout(M, K, I, l->r, true).bytes || !workspace)
      return QLORA_ERR_WORKSPACE;
  }
  if (!dH || !G || !U || !Tg || !Tu || !dG || !dU || !dX || !dAg || !dBg || !dAu || !dBu)
    return QLORA_ERR_NULL;
  if (flags & ~QLORA_BWD_ACCUMULATE_DX) return QLORA_ERR_ARG;
  const void* ptrs[] = {dH, G, U, Tg, Tu, dG, dU, dX, dAg, dBg, dAu, dBu, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return QLORA_ERR_ALIGN;
  // dG and dU feed three products each (the dX GEMM, U = dY B and dB), so the
  // gating backward materialises them; then the two layer backwards, the up
  // projection's adding its dX to the gate's.
  int st = launch_status(qlk::launch_silu_mul_bwd(dH, G, U, M * I, dG, dU, as_stream(stream)));
  if (st) return st;
  st = bwd_common(dG, X, M, K, I, weight(gate->packed, gate->codes, gate->scales, gate->mean, I, K),
                  gate->A, gate->B, gate->r, gate->alpha, Tg, dX, dAg, dBg, flags, workspace,
                  workspace_bytes, stream);
  if (st) return st;
  return bwd_common(dU, X, M, K, I, weight(up->packed, up->codes, up->scales, up->mean, I, K),
                    up->A, up->B, up->r, up->alpha, Tu, dX, dAu, dBu, QLORA_BWD_ACCUMULATE_DX,
                    workspace, workspace_bytes, stream);
}

int silu_mul_fwd(const uint16_t* G, const uint16_t* Up, int64_t n, uint16_t* H, void* stream) {
  if (!G || !Up || !H) return QLORA_ERR_NULL;
  if (n <= 0 || n % 8 != 0 || n / 8 / 256 > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(G) || !aligned16(Up) || !aligned16(H)) return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_silu_mul_fwd(G, Up, n, H, as_stream(stream)));
}

int silu_mul_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* Up, int64_t n,
                 uint16_t* dG, uint16_t* dUp, void* stream) {
  if (!dH || !G || !Up || !dG || !dUp) return QLORA_ERR_NULL;
  if (n <= 0 || n % 8 != 0 || n / 8 / 256 > 0x7fffffff) return QLORA_ERR_SHAPE;
  if (!aligned16(dH) || !aligned16(G) || !aligned16(Up) || !aligned16(dG) || !aligned16(dUp))
    return QLORA_ERR_ALIGN;
  return launch_status(qlk::launch_silu_mul_bwd(dH, G, Up, n, dG, dUp, as_stream(stream)));
}

int nf4_codebook(float* out16) {
  if (!out16) return QLORA_ERR_NULL;
  for (int i = 0; i < 16; ++i) memcpy(&out16[i], &kNF4Bits[i], 4);
  return QLORA_OK;
}

int dq_codebook(float* out256, int* n) {
  if (!out256 || !n) return QLORA_ERR_NULL;
  for (int i = 0; i < 256; ++i) out256[i] = (i < 255) ? (float)(i - 127) / 127.0f : 0.0f;
  *n = 255;
  return QLORA_OK;
}

int dq_float8_codebook(float* out256, int* n) {
  if (!out256 || !n) return QLORA_ERR_NULL;
  for (int i = 0; i < 256; ++i) out256[i] = 0.0f;
  *n = float8_levels(out256);
  return QLORA_OK;
}

const char* qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "null pointer";
    case QLORA_ERR_SHAPE: return "invalid shape";
    case QLORA_ERR_UNSUPPORTED: return "unsupported block size";
    case QLORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_LAUNCH: return "HIP launch failed";
    case QLORA_ERR_ARG: return "invalid argument";
    case QLORA_ERR_SCRATCH: return "needs more scratch memory than the static array holds";
    default: return "unknown status";
  }
}

int qlora_version(void) { return 100; }

}  // extern "C"
