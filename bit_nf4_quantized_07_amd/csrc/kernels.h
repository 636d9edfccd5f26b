// Internal launcher declarations (host side) of the QLoRA NF4 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace qlk {

// A 16-level 4-bit codebook (ascending) and its 15 decision thresholds:
// thr[i] is the exact midpoint of lv[i] and lv[i+1] rounded toward -inf, so
// that "n > thr[i]" <=> "n lies strictly above the midpoint" (ties go to the
// lower index).  NF4 is one instance; the uniform INT4 comparison another.
struct Codebook4 {
  float lv[16];
  float thr[15];
};
Codebook4 make_codebook(const float* levels16);
Codebook4 nf4_codebook4();
// A second-level (8-bit) code table passed as data: n <= 256 ascending levels
// (entries from n on hold 0) and the n - 1 thresholds built the same way.
struct Codebook8 {
  float lv[256];
  float thr[255];
  int n;
};
Codebook8 make_codebook8(const float* levels, int n);

hipError_t launch_nf4_quantize(const float* W, int64_t numel, const Codebook4& cb, uint8_t* packed,
                               float* absmax, hipStream_t st);
// cb8: the second-level table (null: the linear code).
hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* codes, float* scales,
                               float* mean, hipStream_t st, const Codebook8* cb8 = nullptr);
hipError_t launch_nf4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                              const float* mean, int64_t numel, const Codebook4& cb, uint16_t* out,
                              hipStream_t st, const Codebook8* cb8 = nullptr);
hipError_t launch_absmax_dequant(const uint8_t* codes, const float* scales, const float* mean,
                                 int64_t nb, const Codebook8& cb8, float* out, hipStream_t st);
// LoRA dropout: Xd = bf16(x * scale) where Philox4x32-10 keeps the element,
// 0 elsewhere; one mask bit per element.  numel % 32 == 0.
hipError_t launch_lora_dropout(const uint16_t* X, int64_t numel, uint32_t threshold, float scale,
                               uint64_t seed, uint16_t* Xd, uint32_t* mask, hipStream_t st);

// Measurement: caller-owned HIP events recorded on the launch stream around
// individual launches (a null event records nothing; a null Timing times
// nothing).  Passed down per call: the library keeps no timing state.
enum TimedKernel { TK_NONE = 0, TK_FWD_GEMM = 1, TK_DX_GEMM = 2, TK_GEMV = 3, TK_DX_DEQUANT = 4,
                   TK_FWD_DEQUANT = 5, TK_COUNT = 6 };
struct Timing {
  hipEvent_t start[TK_COUNT];
  hipEvent_t stop[TK_COUNT];
};
inline void timer_begin(const Timing* t, int kernel, hipStream_t st) {
  if (t && t->start[kernel]) (void)hipEventRecord(t->start[kernel], st);
}
inline void timer_end(const Timing* t, int kernel, hipStream_t st) {
  if (t && t->stop[kernel]) (void)hipEventRecord(t->stop[kernel], st);
}
// The events of one timed interval recorded by the launches themselves
// (hipExtLaunchKernel): the interval's first kernel records `start` as it
// begins, its last kernel records `stop` as it ends, so the interval holds
// the kernels' execution and no gap of an event record around a launch.
struct Span {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
inline Span span_of(const Timing* t, int kernel) {
  Span s;
  if (t) {
    s.start = t->start[kernel];
    s.stop = t->stop[kernel];
  }
  return s;
}

// Base weight [N, K] as stored: NF4 (packed, codes, scales, mean) or, for
// the unquantised comparison path, plain bf16 (`bf16` non-null, the NF4
// fields unused).
struct NF4Weight {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* scales;
  const float* mean;
  int64_t N, K;
  const uint16_t* bf16 = nullptr;
};

// Token counts up to this take the small-M (GEMV) forward.
constexpr int kGemvMaxM = 16;
// K slices of the small-M T = X A^T partial sums.
constexpr int kTSplits = 16;

// Workspace layout shared by the planner (qlora_workspace_bytes) and the
// launchers, so that both always agree.
struct FwdPlan {
  bool gemv;          // small-M path
  int t_splits;       // contraction splits for T = X A^T
  size_t off_T, off_part, bytes;
  // Split contraction of the register-decode forward when its tiles do not
  // fill the device: K-steps per split (0: none) and the fp32 partials.
  int fwd_kz_len;
  size_t off_fpart;
  // Large M: the forward on a bf16 copy of the weight dequantised once per
  // call (at off_wbf16, 2 N K bytes), read by every token tile.
  bool dequant_fwd;
  size_t off_wbf16;
};
struct BwdPlan {
  int u_splits, t_splits, m_splits_a, m_splits_b;
  bool one_pass_grads;   // dA and dB by launch_adapter_grads (no partials)
  size_t off_U, off_T, off_part, off_part_b, bytes;   // dA partials at off_part, dB at off_part_b
  // dX on a bf16 copy of the weight dequantised once per call (at off_wbf16)
  // instead of decoding every tile in each of the M / 256 token tiles.
  bool dequant_dx;
  size_t off_wbf16;
  // Split contraction of the dX kernel when its tiles do not fill the
  // device: steps per split (0: none) and the fp32 partials.
  int dx_kz_len;
  size_t off_dxpart;
};
// Token count from which the backward dequantises the NF4 weight once.
constexpr int64_t kDequantDxMinM = 1024;
// nf4: the base weight is NF4 (only the NF4 register-decode forward splits
// its contraction); dx: the backward computes dX (its bf16 weight copy and
// split partials are needed only then).
FwdPlan plan_fwd(int64_t M, int64_t K, int64_t N, int r, bool nf4 = true);
BwdPlan plan_bwd(int64_t M, int64_t K, int64_t N, int r, bool dx = true);

// Xa: input of the adapter's down projection (the dropout output); null
// means X itself.
hipError_t launch_qlora_fwd(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                            const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T_out,
                            void* ws, const FwdPlan& plan, hipStream_t st,
                            const uint16_t* Xa = nullptr, const Timing* tm = nullptr);
// Workgroup tile rows walked together by tile_coords (balances the operand
// footprints each XCD keeps in its L2).
int group_for(int tiles_p, int tiles_q, double a_tile_bytes, double b_tile_bytes);
// Y = X W_hat^T + s T B^T for M > kGemvMaxM (T precomputed, bf16 [M, r]);
// supported when K / 64 is a multiple of 4 (else the tile engine runs).
bool fwd_nf4_supported(int64_t K);
// tn_base: the launch covers column tiles (of 128 weight rows) tn_base ..
// of Y only (no split then).
hipError_t launch_fwd_nf4(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* T,
                          const uint16_t* B, int r, float s, uint16_t* Y, hipStream_t st,
                          float* part = nullptr, int kz_len = 0, Span sp = Span(),
                          int tn_base = 0);
// K-steps per split of the forward's contraction for this shape (0: none).
int fwd_split_len(int64_t M, int64_t K, int64_t N);
// Fused gate/up projections of a SiLU-gated MLP (M > kGemvMaxM, K / 64 a
// multiple of 4, both weights [I, K]): G = X Wg^T + sg Tg Bg^T,
// U = X Wu^T + su Tu Bu^T, H = silu(G) U, all bf16 [M, I]; Tg, Tu precomputed.
hipError_t launch_fwd_gated(const uint16_t* X, int64_t M, const NF4Weight& wg, const uint16_t* Tg,
                            const uint16_t* Bg, int rg, float sg, const NF4Weight& wu,
                            const uint16_t* Tu, const uint16_t* Bu, int ru, float su, uint16_t* G,
                            uint16_t* U, uint16_t* H, hipStream_t st);
// The gated MLP's gate/up forward in one kernel (with the two T launches
// before it), taken when mlp_fwd_fused(M, K, I); the caller composes the two
// layer forwards and the gating otherwise (also where each projection runs
// the wide tile on a dequantised copy, which beats the fused tile).  Needs no
// workspace.
struct LoraLinear {
  NF4Weight w;
  const uint16_t* A;
  const uint16_t* B;
  int r;
  float s;
};
bool mlp_fwd_fused(int64_t M, int64_t K, int64_t I);
hipError_t launch_mlp_fwd(const uint16_t* X, int64_t M, const LoraLinear& gate,
                          const LoraLinear& up, uint16_t* G, uint16_t* U, uint16_t* H,
                          uint16_t* Tg, uint16_t* Tu, hipStream_t st);
// dX = dY W_hat (+ s U A) for N a multiple of 256 (else the tile engine runs).
bool dx_nf4_supported(int64_t N);
// With a dropout mask (bit per element of dX, row-major), the adapter term
// becomes mask * keep_scale * s U A.
hipError_t launch_dx_nf4(const uint16_t* dY, int64_t M, const NF4Weight& w, const uint16_t* U,
                         const uint16_t* A, int r, float s, uint16_t* dX, bool accumulate,
                         hipStream_t st, const uint32_t* mask = nullptr, float keep_scale = 1.0f,
                         float* part = nullptr, int kz_len = 0, Span sp = Span());
// Steps per split of the dX kernel's contraction for this shape (0: none).
int dx_split_len(int64_t M, int64_t K, int64_t N);
// out (bf16, stride values per split) = the fixed-order sum of the fp32
// split partials, plus out's own values when accumulating; one rounding.
hipError_t launch_split_reduce(const float* part, int splits, int64_t stride, uint16_t* out,
                               bool accumulate, hipStream_t st, hipEvent_t stop = nullptr);
// dX (+)= bf16(mask * keep_scale * s U A): the adapter term alone, for the
// tile-engine fallback of the dropout backward.
hipError_t launch_dx_adapter_masked(const uint16_t* U, const uint16_t* A, int64_t M, int64_t K,
                                    int r, float s, const uint32_t* mask, float keep_scale,
                                    uint16_t* dX, bool accumulate, hipStream_t st);
// out = S W^T (as launch_rank16: W = [r, C] or, transposed, [C, r]) and the
// dequantisation of w into wout (bf16 [N, K], as launch_nf4_dequant), in one
// launch: the backward's U = dY B, the wide forward's T = X A^T.
hipError_t launch_rank16_and_dequant(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W,
                                     bool transposed, int r, uint16_t* out, const NF4Weight& w,
                                     uint16_t* wout, hipStream_t st, Span sp = Span());
// Y = X wb^T + s T B^T on a bf16 weight wb [N, K] with 256 x 256 tiles of
// four 128 x 128 waves (the wide dX tile in its forward form), in the
// register-decoded forward's contraction order; for shapes where
// fwd_wide_bf16_fits.
// It covers the first `cols` 256-wide column tiles of Y (its weight rows
// below 256 cols are read); fwd_wide_columns(M, N) is the count after which
// the register-decoded tile (launch_fwd_nf4 with a first column tile) takes
// the rest in fewer rounds of the device.
bool fwd_wide_bf16_fits(int64_t M, int64_t K, int64_t N);
int fwd_wide_columns(int64_t M, int64_t N);
hipError_t launch_fwd_wide_bf16(const uint16_t* X, int64_t M, const uint16_t* wb, int64_t N,
                                int64_t K, const uint16_t* T, const uint16_t* B, int r, float s,
                                uint16_t* Y, int cols, hipStream_t st, Span sp = Span());
// Y = X wb^T + s T B^T on a bf16 base weight wb [N, K] (the dX kernel in its
// forward form), for K a multiple of 256.
hipError_t launch_fwd_bf16(const uint16_t* X, int64_t M, const uint16_t* wb, int64_t N, int64_t K,
                           const uint16_t* T, const uint16_t* B, int r, float s, uint16_t* Y,
                           hipStream_t st);
// dA = s U^T X ([r, K], fp32) and dB = s dY^T T ([N, r], fp32) in one launch
// that contracts over all M tokens per output column slice (no partial sums);
// for the shapes adapter_grads_supported accepts (r a multiple of 8, at most
// 64; every operand under 2 GiB).
bool adapter_grads_supported(int64_t M, int64_t K, int64_t N, int r);
hipError_t launch_adapter_grads(const uint16_t* U, const uint16_t* X, const uint16_t* dY,
                                const uint16_t* T, int64_t M, int64_t K, int64_t N, int r,
                                float s, float* dA, float* dB, hipStream_t st);
// out[M, r] (bf16) = S[M, C] W^T with W = [r, C] or, transposed, [C, r].
hipError_t launch_rank16(const uint16_t* S, int64_t M, int64_t C, const uint16_t* W, bool transposed,
                         int r, uint16_t* out, hipStream_t st);
hipError_t launch_gemv(const uint16_t* X, int64_t M, const NF4Weight& w, const uint16_t* A,
                       const uint16_t* B, int r, float s, uint16_t* Y, uint16_t* T, float* Tpart,
                       hipStream_t st, const uint16_t* Xa = nullptr, const Timing* tm = nullptr);
// X is the adapter input (the dropout output Xd when mask is non-null): it
// feeds T (when not given) and dA.  mask/keep_scale: dropout of the adapter
// input, applied to the adapter term of dX.
hipError_t launch_qlora_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, const NF4Weight& w,
                            const uint16_t* A, const uint16_t* B, int r, float s,
                            const uint16_t* T, uint16_t* dX, float* dA, float* dB,
                            bool accumulate_dx, void* ws, const BwdPlan& plan, hipStream_t st,
                            const uint32_t* mask = nullptr, float keep_scale = 1.0f,
                            const Timing* tm = nullptr);


// W_merged = bf16(w_hat + s B A), bf16 [N, K].
hipError_t launch_merge(const NF4Weight& w, const uint16_t* A, const uint16_t* B, int r, float s,
                        uint16_t* out, hipStream_t st);

// dst [rows_dst, cols_dst] = src [rows_src, cols_src] zero-extended or cut
// (row-major, contiguous): adapter-rank padding at the boundary.
hipError_t launch_pad2d(const uint16_t* src, int64_t rows_src, int64_t cols_src, uint16_t* dst,
                        int64_t rows_dst, int64_t cols_dst, hipStream_t st);
hipError_t launch_pad2d(const float* src, int64_t rows_src, int64_t cols_src, float* dst,
                        int64_t rows_dst, int64_t cols_dst, hipStream_t st);

hipError_t launch_silu_mul_fwd(const uint16_t* G, const uint16_t* U, int64_t n, uint16_t* H,
                               hipStream_t st);
hipError_t launch_silu_mul_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* U,
                               int64_t n, uint16_t* dG, uint16_t* dU, hipStream_t st);

}  // namespace qlk
