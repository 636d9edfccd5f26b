/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA NF4 linear-layer library.
 *
 * The library implements the QLoRA linear layer of
 *     h = dequant(W0_NF4) x + (alpha / r) B A x
 * (llm-compass "QLoRA", section 方法与公式, the displayed equation), forward and
 * backward, with the frozen base weight stored as 4-bit NormalFloat codes in
 * blocks of 64 and double-quantised block constants (aigrafen.se "QLoRA",
 * list "Tre tekniska bitar" items 1-2; auryth.ai "QLoRA", "Hoe het werkt"
 * NF4 and Dubbele Quantisatie boxes; llm-compass 方法与公式 items 1-2).
 *
 * Conventions for every call
 *   - Array pointers are DEVICE pointers into caller-owned, contiguous,
 *     row-major buffers, each 16-byte aligned (the kernels use 128-bit loads).
 *   - bf16 values travel as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns immediately.
 *   - Outputs are overwritten (never accumulated) unless a flag says
 *     otherwise.  The library allocates no device memory: scratch space comes
 *     from the caller's `workspace`.  It holds no mutable state, so calls on
 *     different streams with different workspaces may run concurrently; two
 *     calls that share a workspace must be ordered (e.g. on one stream).
 *   - Calls return a status code (QLORA_* below).  All argument checks run on
 *     the host before any launch, so a non-zero status means nothing was
 *     enqueued.  Faults inside a kernel surface at the next stream
 *     synchronisation, as in any HIP program.  No C++ exception crosses this
 *     interface and the library prints nothing.
 *
 * Storage format (all produced by nf4_quantize + double_quant):
 *   W0       [N, K] fp32, row-major (out x in), K % 64 == 0
 *   packed   [N*K/2] uint8: element 2j in the HIGH nibble of byte j
 *   absmax   [N*K/64] fp32: max |w| of each run of 64 consecutive elements
 *   codes    [N*K/64] uint8: 8-bit code of each centred constant
 *   scales   [ceil(N*K/64/256)] fp32: one second-level scale per 256 constants
 *   mean     [1] fp32 (device): mean of all absmax values of the tensor
 * Dequantised weight: w_hat = fp32(Q4[nibble] * a_hat),
 *   a_hat = fp32(fp32(Q8[code] * scale) + mean),  Q8[i] = fp32(i-127)/127.
 */
#ifndef QLORA_H_
#define QLORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QLORA_OK                 0
#define QLORA_ERR_NULL          -1  /* a required pointer is NULL                   */
#define QLORA_ERR_SHAPE         -2  /* M,N,K <= 0; K % 64; N % 8; r outside [1, 256];
                                       N*K odd or too large; an operand >= 2 GiB      */
#define QLORA_ERR_UNSUPPORTED   -3  /* blocksize != 64 or dq_blocksize != 256       */
#define QLORA_ERR_ALIGN         -4  /* a pointer is not 16-byte aligned             */
#define QLORA_ERR_WORKSPACE     -5  /* workspace NULL or smaller than required      */
#define QLORA_ERR_LAUNCH        -6  /* the HIP runtime refused a launch             */
#define QLORA_ERR_ARG           -7  /* other invalid argument (alpha not finite,
                                       unknown flag bits, p outside [0, 1), a
                                       codebook not finite and ascending)            */
#define QLORA_ERR_SCRATCH       -8  /* qlora_linear_bwd_noalloc: the call needs more
                                       than QLORA_NOALLOC_SCRATCH_BYTES of scratch   */

/* qlora_linear_bwd flag: add the computed dX into the bf16 values already in
 * dX instead of overwriting them (used when two linears share an input, as
 * the gate and up projections of a gated MLP do). */
#define QLORA_BWD_ACCUMULATE_DX  1

/* ---- quantisation (run once, when the base weight is loaded) ------------ */

/* Blockwise NF4 quantisation of W0 [N, K].
 * llm-compass "QLoRA", 方法与公式 item 1: blocks of 64 weights, one absmax
 * constant each; auryth.ai "QLoRA", NF4 box: 16 levels at normal quantiles.
 * For each block: absmax = max |w|; n = w / absmax (IEEE fp32 division);
 * code = index of the nearest NF4 level, ties to the lower index; a block of
 * zeros gets the zero level (index 7).  Non-finite inputs give unspecified
 * codes.  Bit-exact: same bytes on every run.
 * In:  W0 fp32 [N*K].   Out: packed uint8 [N*K/2], absmax fp32 [N*K/64].
 * Requires K % 64 == 0, blocksize == 64. */
int nf4_quantize(const float* W0, int64_t N, int64_t K, int blocksize,
                 uint8_t* packed, float* absmax, void* stream);

/* Double quantisation of the block constants.
 * aigrafen.se "QLoRA" item 2 and llm-compass 方法与公式 item 2: the fp32
 * constants are quantised again, to 8 bits.  mean = fp32(S / nblocks) with S
 * the fp64 sum taken sequentially inside each run of 256 constants and then
 * sequentially over those partial sums; c = fp32(absmax - mean); per run of
 * 256: scale = max |c|; code = nearest level of Q8 to fp32(c / scale), ties
 * to the lower index (scale == 0 gives code 127).
 * In:  absmax fp32 [nblocks].
 * Out: codes uint8 [nblocks], scales fp32 [ceil(nblocks/256)], mean fp32 [1].
 * Requires dq_blocksize == 256.  Bit-exact. */
int double_quant(const float* absmax, int64_t nblocks, int dq_blocksize,
                 uint8_t* codes, float* scales, float* mean, void* stream);

/* Dequantise to the bf16 compute type (auryth.ai "QLoRA", DATASTROOM box;
 * llm-compass 直觉与动机).  W_bf16[i] = RNE_bf16(w_hat[i]).  Bit-exact.
 * Out: W_bf16 uint16 [N*K]. */
int nf4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                const float* mean, int64_t N, int64_t K, int blocksize,
                int dq_blocksize, uint16_t* W_bf16, void* stream);

/* ---- other 4-bit codebooks through the same kernels ---------------------- */

/* Blockwise quantisation onto any ascending 16-level codebook, with the NF4
 * rules (absmax per 64, n = w / absmax, nearest level with ties to the lower
 * index, n = 0 for an all-zero block).  For the comparison the pages draw
 * between NF4 and uniform INT4, whose evenly spaced levels waste resolution
 * where normal weights are dense (learn-interview-questions §2, "4-bit
 * NormalFloat (NF4) vs. Standard INT4"; llm-compass 方法与公式 item 1).
 *   levels  HOST memory, 16 finite fp32 values, strictly ascending
 * Decision thresholds are the exact midpoints rounded toward -inf.  Same
 * outputs, sizes and rules as nf4_quantize (which is this call with the NF4
 * levels); QLORA_ERR_ARG for a codebook that is not finite and ascending.
 * Bit-exact. */
int codebook_quantize(const float* W0, int64_t N, int64_t K, int blocksize,
                      const float* levels, uint8_t* packed, float* absmax, void* stream);

/* Dequantisation with the same codebook: W_bf16[i] = RNE_bf16(fp32(
 * levels[nibble] * a_hat)), a_hat as in nf4_dequant.  Bit-exact. */
int codebook_dequant(const uint8_t* packed, const uint8_t* codes, const float* scales,
                     const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                     const float* levels, uint16_t* W_bf16, void* stream);

/* ---- other 8-bit codes for the second level ------------------------------ */

/* The pages give the second level only as "8 bits" (auryth.ai "QLoRA",
 * Dubbele Quantisatie box; llm-compass "QLoRA", 方法与公式 item 2).  The layer
 * uses the linear code Q8[i] = (i - 127) / 127; these calls take any
 * second-level table as data, e.g. the 8-bit-float table of
 * dq_float8_codebook, whose levels are dense near zero, so the ordinary
 * constants of a group whose scale an outlier sets keep their precision.
 *   levels   HOST memory, 2 <= nlevels <= 256 finite values, strictly
 *            ascending (QLORA_ERR_ARG otherwise); code byte = index
 * Rules as double_quant (mean, centring, per-256 scale, nearest level with
 * ties to the lower index; a group with scale 0 gets the level nearest 0).
 * Bit-exact; with the linear table the codes equal double_quant's. */
int double_quant_table(const float* absmax, int64_t nblocks, int dq_blocksize,
                       const float* levels, int nlevels, uint8_t* codes, float* scales,
                       float* mean, void* stream);

/* a_hat[b] = fp32(fp32(levels[codes[b]] * scales[b / 256]) + mean), fp32
 * [nblocks] (codes from nlevels on read 0).  Bit-exact. */
int absmax_dequant(const uint8_t* codes, const float* scales, const float* mean,
                   int64_t nblocks, int dq_blocksize, const float* levels, int nlevels,
                   float* out, void* stream);

/* nf4_dequant (or codebook_dequant with levels4; NULL = NF4) with the second
 * level decoded from levels8.  Bit-exact. */
int dequant_tables(const uint8_t* packed, const uint8_t* codes, const float* scales,
                   const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                   const float* levels4, const float* levels8, int nlevels8, uint16_t* W_bf16,
                   void* stream);

/* ---- the linear layer --------------------------------------------------- */

/* Forward  Y = X W_hat^T + s (X A^T) B^T,  s = fp32(alpha / r)
 * (llm-compass 方法与公式, the equation, for a batch of rows).
 *   X  bf16 [M, K]     activations
 *   A  bf16 [r, K]     adapter down-projection
 *   B  bf16 [N, r]     adapter up-projection
 *   Y  bf16 [M, N]     output
 *   T_out bf16 [M, r]  optional: X A^T for the backward (NULL = not stored)
 * Below 256 output tiles of 256 x 256, W_hat is never written to memory:
 * tiles are dequantised on the fly.  From 256 such tiles (e.g. 4096 tokens
 * and 4096 outputs), with K % 128 == 0 and 2 N K < 2 GiB, the weight is
 * dequantised once per call into the workspace (2 N K bytes of it, next to
 * T = X A^T in the same launch) and a wide bf16 tile reads that copy (the
 * pages' dequantise-then-matmul, llm-compass 直觉与动机); where the wide
 * tiles' last round would only part-fill the device, the on-the-fly tile
 * takes the last columns.  With K % 256 == 0 the two tiles give the same
 * bits.  Accumulation is fp32; Y is rounded to bf16 once.  When Y has fewer than
 * 128 tiles of 256 tokens x 128 outputs, the contraction over K is split
 * into ranges whose fp32 partials pass through the workspace and are added
 * in a fixed order: still deterministic, though the bits can differ from a
 * shape that does not split.  Results meet
 * |err|_F / |ref|_F <= 1e-2 and max|err| <= 3e-2 max|ref| against an exact
 * evaluation of the same bf16 inputs.
 * Requires 1 <= M, K % 64 == 0, N % 8 == 0 (every row of X, Y, dY and dX
 * starts on a 16-byte boundary: the kernels move rows in 128-bit pieces),
 * 1 <= r <= 256, each of X, Y (2 M K, 2 M N bytes) and the packed weight
 * (N K / 2 bytes) under 2 GiB, and workspace_bytes >=
 * qlora_workspace_bytes(M, K, N, r, 0).  A rank that is not a multiple of 8
 * runs as the next multiple of 8 on zero-padded copies of A and B in the
 * workspace (the kernels read adapter rows in 16-byte pieces); the padding
 * adds only exact zeros, and s stays alpha / r. */
int qlora_linear_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                     const uint8_t* packed, const uint8_t* codes, const float* scales,
                     const float* mean, const uint16_t* A, const uint16_t* B,
                     int r, float alpha, uint16_t* Y, uint16_t* T_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the forward above.  Gradients reach the adapters only; the
 * frozen base weight gets none (aigrafen.se "QLoRA", opening paragraph;
 * llm-compass 方法与公式, text under the equation; skillbyai "Quantized base
 * plus LoRA").  With U = dY B:
 *   dX = dY W_hat + s U A      bf16 [M, K]  (NULL = skip)
 *   dA = s U^T X               fp32 [r, K]
 *   dB = s dY^T (X A^T)        fp32 [N, r]
 * T is the X A^T saved by the forward (bf16 [M, r]); NULL = recompute it.
 * flags: 0 or QLORA_BWD_ACCUMULATE_DX.  The reductions over M run in a fixed
 * order, so repeated calls give identical bits: for r <= 64 one workgroup
 * per 32 output columns of dA^T or dB contracts over all M tokens (no
 * partial sums in the workspace); above, fp32 partials over token ranges go
 * through the workspace and are added in index order.  Same shape rules and
 * tolerances as the forward; workspace >= qlora_workspace_bytes(..., 1).
 * For M >= 1024 (and N % 256 == 0, 2 N K < 2 GiB) the weight is dequantised
 * once per call into the workspace (2 N K bytes of it) and dX runs on that
 * bf16 copy (the pages' dequantise-then-matmul, llm-compass 直觉与动机): the
 * same bits as decoding in every tile with the same split of the
 * contraction, without decoding it again for every 256 tokens.  dX splits
 * its contraction over N like the forward when its tiles (256 tokens x 128
 * features) number fewer than 128. */
int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K, int64_t N,
                     const uint8_t* packed, const uint8_t* codes, const float* scales,
                     const float* mean, const uint16_t* A, const uint16_t* B,
                     int r, float alpha, const uint16_t* T,
                     uint16_t* dX, float* dA, float* dB, int flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/* qlora_linear_bwd for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments without the workspace, the same kernels and bit-identical
 * results.  Its scratch memory is a static device array of
 * QLORA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds from
 * module load until the process ends; the call allocates nothing.  Shapes
 * whose backward needs more scratch than that (qlora_workspace_bytes(M, K, N,
 * r, 1), less the dX parts when dX is NULL) return QLORA_ERR_SCRATCH before
 * anything is launched; 64 MiB holds the backward of a 4096 x 4096 layer at
 * 2048 tokens.  All calls on one GPU share the array: two calls that overlap
 * on the same GPU (different streams, no ordering between them) race. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int qlora_linear_bwd_noalloc(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K,
                             int64_t N, const uint8_t* packed, const uint8_t* codes,
                             const float* scales, const float* mean, const uint16_t* A,
                             const uint16_t* B, int r, float alpha, const uint16_t* T, uint16_t* dX,
                             float* dA, float* dB, int flags, void* stream);

/* The same layer with an unquantised bf16 base weight W [N, K] (bf16,
 * row-major): the comparison the pages draw between LoRA on a bf16 base and
 * QLoRA, where QLoRA trains 20-40 % slower per step because of the
 * dequantisation in every forward pass (aigrafen.se "QLoRA", paragraph
 * "Priset"; llm-compass "QLoRA", 与 baseline 对比 table, row 训练速度).  The
 * backward runs the same kernels with the dequantisation switched off, the
 * forward (K a multiple of 256, more than 16 tokens) the dX kernel's forward
 * form, a bf16 GEMM; everything else (adapter branch, reductions,
 * tolerances, workspace size) is as in qlora_linear_fwd / qlora_linear_bwd,
 * with W_hat = W.  Requires W under
 * 2 GiB (2 N K bytes) in addition to their shape rules. */
int qlora_linear_fwd_bf16(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                          const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* Y,
                          uint16_t* T_out, void* workspace, size_t workspace_bytes, void* stream);
int qlora_linear_bwd_bf16(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K, int64_t N,
                          const uint16_t* W, const uint16_t* A, const uint16_t* B, int r,
                          float alpha, const uint16_t* T, uint16_t* dX, float* dA, float* dB,
                          int flags, void* workspace, size_t workspace_bytes, void* stream);

/* ---- LoRA dropout on the adapter input ---------------------------------- */

/* Every training recipe on the pages sets lora_dropout = 0.05 (aigrafen.se
 * "QLoRA", code block; llm-compass "QLoRA", code under 实现要点; skillbyai
 * "A QLoRA setup in outline"; learn-interview-questions §3): elements of the
 * input of A are dropped and the rest scaled by 1/(1-p); the base sees X.
 *
 * lora_dropout draws the mask and writes the dropped input:
 *   element i of the row-major X [M, K] is kept iff word i % 4 of
 *   Philox4x32-10(counter = (g mod 2^32, g div 2^32, 0, 0),
 *                 key = (seed mod 2^32, seed div 2^32)),  g = i div 4,
 *   is >= floor(p * 2^32)  (Salmon et al., "Parallel random numbers: as easy
 *   as 1, 2, 3", SC 2011; a pure function of (seed, i));
 *   Xd[i] = kept ? RNE_bf16(fp32(x * fp32(1/(1-p)))) : +0      bf16 [M, K]
 *   mask[i / 32] bit (i % 32) = kept                           uint32 [M*K/32]
 * Requires 0 <= p < 1, M >= 1, K % 32 == 0, X and Xd under 2 GiB.  Bit-exact.
 * Use a fresh seed per step and layer. */
int lora_dropout(const uint16_t* X, int64_t M, int64_t K, double p, uint64_t seed,
                 uint16_t* Xd, uint32_t* mask, void* stream);

/* Forward with the dropped adapter input:
 *   Y = X W_hat^T + s (Xd A^T) B^T,   T_out = Xd A^T
 * Xd bf16 [M, K] from lora_dropout; everything else as qlora_linear_fwd. */
int qlora_linear_fwd_dropout(const uint16_t* X, const uint16_t* Xd, int64_t M, int64_t K,
                             int64_t N, const uint8_t* packed, const uint8_t* codes,
                             const float* scales, const float* mean, const uint16_t* A,
                             const uint16_t* B, int r, float alpha, uint16_t* Y,
                             uint16_t* T_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Backward of qlora_linear_fwd_dropout, the mask held fixed.  With U = dY B:
 *   dX = dY W_hat + (s U A) * mask * fp32(1/(1-p))     bf16 [M, K]
 *   dA = s U^T Xd,   dB = s dY^T (Xd A^T)               fp32
 * T = Xd A^T from the forward (NULL = recompute from Xd); mask and p as given
 * to lora_dropout.  Flags, workspace, shape rules and tolerances as in
 * qlora_linear_bwd. */
int qlora_linear_bwd_dropout(const uint16_t* dY, const uint16_t* Xd, const uint32_t* mask,
                             double p, int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                             const uint8_t* codes, const float* scales, const float* mean,
                             const uint16_t* A, const uint16_t* B, int r, float alpha,
                             const uint16_t* T, uint16_t* dX, float* dA, float* dB, int flags,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace the forward (is_bwd = 0) or backward (is_bwd = 1)
 * needs for these sizes; 0 means none.  Returns 0 for invalid sizes too. */
size_t qlora_workspace_bytes(int64_t M, int64_t K, int64_t N, int r, int is_bwd);

/* ---- fused gate/up projections of a SiLU-gated MLP ---------------------- */

/* One QLoRA linear of the MLP: NF4 base [I, K] as nf4_quantize + double_quant
 * store it (device pointers), bf16 adapters A [r, K] and B [I, r] (device),
 * r and alpha as in qlora_linear_fwd.  Passed by HOST pointer. */
typedef struct qlora_lora_linear {
  const uint8_t* packed;
  const uint8_t* codes;
  const float* scales;
  const float* mean;
  const uint16_t* A;
  const uint16_t* B;
  int r;
  float alpha;
} qlora_lora_linear;

/* The gate and up projections of a SiLU-gated MLP with LoRA on both (the
 * pages put adapters on gate_proj and up_proj as on every linear, aigrafen.se
 * "QLoRA", code block, target_modules) and the gating, in one pass over X:
 *   G = X Wg^T + sg (X Ag^T) Bg^T,   U = X Wu^T + su (X Au^T) Bu^T,
 *   H = silu(G) * U,   silu(g) = g / (1 + exp(-g))
 *   X  bf16 [M, K];   G, U, H  bf16 [M, I];   Tg, Tu  bf16 [M, rg], [M, ru]
 * G, U, Tg and Tu are what the backward needs.  G and U are bit-identical to
 * qlora_linear_fwd on each projection and H to silu_mul_fwd(G, U).  For
 * M > 16, K % 256 == 0 and both ranks multiples of 8, one kernel computes G
 * and U tile by tile and writes H from the same tile (no second pass over G
 * and U) and needs no workspace; other shapes, and those where
 * qlora_linear_fwd dequantises the weight once (see there; faster than the
 * fused tile), run the two layer forwards and the elementwise gating.
 * Requires the shape rules of qlora_linear_fwd for each projection (I plays
 * N), both weights [I, K], and workspace_bytes >= qlora_workspace_bytes(M, K,
 * I, r, 0) for both r (always sufficient). */
int qlora_mlp_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t I,
                  const qlora_lora_linear* gate, const qlora_lora_linear* up,
                  uint16_t* G, uint16_t* U, uint16_t* H, uint16_t* Tg, uint16_t* Tu,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Backward of qlora_mlp_fwd from dH = dL/dH, in one call:
 *   dG = dH * U * sig(G) * (1 + G (1 - sig(G))),  dU = dH * silu(G)   (silu_mul_bwd)
 *   dX = dG Wg + sg (dG Bg) Ag + dU Wu + su (dU Bu) Au          bf16 [M, K]
 *   dAg, dBg, dAu, dBu as qlora_linear_bwd gives them for each projection.
 * G, U, Tg, Tu are the forward's; dG and dU (bf16 [M, I], caller-owned) are
 * written on the way, since they feed three products each (the dX GEMM, U =
 * dY B and dB).  The gate's dX is written (or, with QLORA_BWD_ACCUMULATE_DX,
 * added) and the up projection's is added to it; the results are those of
 * silu_mul_bwd followed by the two qlora_linear_bwd calls.  Shape rules as
 * qlora_mlp_fwd; workspace_bytes >= qlora_workspace_bytes(M, K, I, r, 1) for
 * both r. */
int qlora_mlp_bwd(const uint16_t* dH, const uint16_t* X, int64_t M, int64_t K, int64_t I,
                  const qlora_lora_linear* gate, const qlora_lora_linear* up,
                  const uint16_t* G, const uint16_t* U, const uint16_t* Tg, const uint16_t* Tu,
                  uint16_t* dG, uint16_t* dU, uint16_t* dX, float* dAg, float* dBg,
                  float* dAu, float* dBu, int flags, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ---- serving: fold the adapter into the base ---------------------------- */

/* W_merged = RNE_bf16( w_hat_bf16 + s (B A) ),  s = fp32(alpha / r).
 * A 4-bit base must be dequantised before an adapter can be merged into it,
 * and the merged weight keeps the base's quantisation error (llm-compass
 * "QLoRA", 与 baseline 对比 table, row 部署合并, and 实现要点, the item on
 * merging; auryth.ai "QLoRA", FAQ, the question on inference; skillbyai
 * "QLoRA: Fine-Tuning on One Consumer GPU", "Quantized base plus LoRA").
 *   w_hat_bf16  the weight nf4_dequant produces (same bits)
 *   A  bf16 [r, K],  B  bf16 [N, r]
 *   W_merged  bf16 [N, K] (caller-owned, overwritten)
 * B A is accumulated in fp32 (MFMA), added with one fp32 fused multiply-add
 * and rounded to bf16 once; each value is within one bf16 rounding step of
 * the exactly evaluated merge.
 * Requires K % 64 == 0, N % 8 == 0, 1 <= r <= 256, blocksize == 64,
 * dq_blocksize == 256, finite alpha. */
int qlora_merge(const uint8_t* packed, const uint8_t* codes, const float* scales,
                const float* mean, int64_t N, int64_t K, int blocksize, int dq_blocksize,
                const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* W_merged,
                void* stream);

/* ---- gated-MLP glue (not a QLoRA step; used by MLP workloads) ----------- */

/* H = silu(G) * Up, silu(g) = g / (1 + exp(-g)); bf16 [n] each, n % 8 == 0. */
int silu_mul_fwd(const uint16_t* G, const uint16_t* Up, int64_t n, uint16_t* H,
                 void* stream);

/* dG = dH * Up * sig(G) * (1 + G (1 - sig(G))),  dUp = dH * silu(G). */
int silu_mul_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* Up, int64_t n,
                 uint16_t* dG, uint16_t* dUp, void* stream);

/* ---- measurement ---------------------------------------------------------- */

/* Internal kernels that can be timed individually. */
#define QLORA_KERNEL_FWD_GEMM   1  /* fused dequant GEMM  Y = X W_hat^T + s T B^T     */
#define QLORA_KERNEL_DX_GEMM    2  /* fused dequant GEMM  dX = dY W_hat + s U A       */
#define QLORA_KERNEL_GEMV       3  /* small-M dequant GEMV forward                    */
#define QLORA_KERNEL_DX_DEQUANT 4  /* the backward's one-off dequantisation (M >= 1024),
                                       launched together with U = dY B                 */
#define QLORA_KERNEL_FWD_DEQUANT 5 /* the forward's one-off dequantisation (wide shapes),
                                       launched together with T = X A^T                */
#define QLORA_KERNEL_COUNT      6

/* Caller-owned HIP events (hipEvent_t as void*), indexed by the kernel ids
 * above (slot 0 unused).  In a timed call, start[k] marks the beginning of
 * kernel k's execution and stop[k] its end (with a split contraction, the end
 * of the reduction that follows it): the dedicated kernels record the events
 * as part of their own launch (hipExtLaunchKernel), the generic tile engine
 * has them recorded on the stream right before and after its launch.  NULL
 * slots record nothing.  The struct is read during the call only. */
typedef struct qlora_timing {
  void* start[QLORA_KERNEL_COUNT];
  void* stop[QLORA_KERNEL_COUNT];
} qlora_timing;

/* qlora_linear_fwd / qlora_linear_bwd with the execution of their dominant
 * kernels marked by the caller's events (for benchmarks: events between two
 * kernels can delay the second one's dispatch, so a step's own time is best
 * taken from untimed calls).  Same arguments, results and status codes;
 * timing == NULL makes them the plain calls. */
int qlora_linear_fwd_timed(const uint16_t* X, int64_t M, int64_t K, int64_t N,
                           const uint8_t* packed, const uint8_t* codes, const float* scales,
                           const float* mean, const uint16_t* A, const uint16_t* B, int r,
                           float alpha, uint16_t* Y, uint16_t* T_out, void* workspace,
                           size_t workspace_bytes, void* stream, const qlora_timing* timing);
int qlora_linear_bwd_timed(const uint16_t* dY, const uint16_t* X, int64_t M, int64_t K,
                           int64_t N, const uint8_t* packed, const uint8_t* codes,
                           const float* scales, const float* mean, const uint16_t* A,
                           const uint16_t* B, int r, float alpha, const uint16_t* T, uint16_t* dX,
                           float* dA, float* dB, int flags, void* workspace,
                           size_t workspace_bytes, void* stream, const qlora_timing* timing);

/* ---- host-side helpers --------------------------------------------------- */

/* The 16 NF4 levels the kernels use (HOST memory, 16 floats). */
int nf4_codebook(float* out16);

/* The 8-bit levels the kernels use (HOST memory, 256 floats; *n = 255). */
int dq_codebook(float* out256, int* n);

/* The 8-bit-float second-level table (HOST memory, 256 floats; *n = 253):
 * every finite value of the 8-bit float with 4 exponent bits (bias 7) and 3
 * mantissa bits, divided by its largest value 448 (each quotient rounded once
 * to fp32), ascending, zero at index 126; entries from 253 on are 0. */
int dq_float8_codebook(float* out256, int* n);

/* Static text for a status code. */
const char* qlora_strerror(int status);

/* Library version, e.g. 100 for 0.1.0. */
int qlora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H_ */
