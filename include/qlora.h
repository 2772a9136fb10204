/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA frozen-base linear layer.
 *
 * The layer keeps a frozen base weight in 4-bit NF4 with double-quantised
 * block scales and adds a full-precision LoRA path:
 *
 *     y = x . deq(W)^T + (alpha/r) . (x . A^T) . B^T
 *
 * Sources, cited by page title and section:
 *   [QLoRA / infivelines.com]  NF4 levels at normal quantiles; one scale per
 *       block of 64 weights; the scales quantised again in blocks of 256
 *       (~0.127 bits/weight); dequantised to bf16 one block at a time
 *       inside the matrix multiply; gradients pass through the frozen base.
 *   [QLoRA -- the democratization event, the recipe]  4-bit NF4 frozen
 *       base, 16-bit adapters, dequantised on the fly, gradients into the
 *       adapters only; double quantisation of the block scale factors.
 *   [QLoRA -- Module 12.4, "Design Details That Matter" / "Hugging Face +
 *       BitsAndBytes"]  NF4, double quant; LoraConfig(r, lora_alpha).
 *   [QLoRA, and fine-tuning a 7B model on a free GPU, "What each setting is
 *       doing"]  stored in 4 bits, computed in bfloat16, dequantised for
 *       each matrix multiply.
 *   The pages defer the LoRA equation; the form above with s = alpha/r is
 *   the standard LoRA layer the pages configure.
 *
 * Conventions (all entry points)
 *   - Plain C types only.  bf16 tensors are passed as uint16_t bit patterns.
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Every pointer argument except where noted is a DEVICE pointer, owned
 *     and allocated by the caller, 16-byte aligned, row-major and densely
 *     packed.  The library allocates no device memory and keeps no state
 *     between calls except its constant NF4 table.
 *   - Inputs are never written.  Outputs are fully overwritten (dA/dB are
 *     accumulated into when `accumulate` is nonzero).  Outputs must not
 *     alias inputs or each other.
 *   - Return value: QLORA_OK (0) means the work was enqueued on `stream`;
 *     a negative status means nothing was enqueued.  Argument validation
 *     happens before any HIP call.  Device-side faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 *   - Inputs must be finite (no NaN/Inf); this is not checked.
 *   - Calls on the same stream are ordered; the workspace of a call may be
 *     reused by the next call on the same stream.  Concurrent calls on
 *     different streams need separate workspaces.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define QLORA_OK          0
#define QLORA_EINVAL     (-1) /* null pointer, negative size, aliasing        */
#define QLORA_ESHAPE     (-2) /* K or N not a multiple of 64, r > 256 or r%8,
                                  or a tensor at or above 2 GiB (see below)    */
#define QLORA_EALIGN     (-3) /* a device pointer is not 16-byte aligned      */
#define QLORA_ENOTSUP    (-4) /* blocksize != 64 or blocksize2 != 256         */
#define QLORA_EWORKSPACE (-5) /* workspace NULL or smaller than required      */
#define QLORA_EHIP       (-6) /* a HIP launch or runtime call failed          */
#define QLORA_ESCRATCH   (-7) /* the allocation-free call needs more than
                                  QLORA_NOALLOC_SCRATCH_BYTES of scratch       */

#define QLORA_BLOCK   64   /* weights per absmax block                       */
#define QLORA_GROUP   256  /* block scales per double-quantisation group      */
#define QLORA_MAX_RANK 256

/* A frozen NF4 base weight W [N, K] (out_features x in_features, row-major).
 * All pointers are device pointers owned by the caller.
 *   codes   [N*K/2]           byte j = code(2j) | code(2j+1) << 4
 *   qscale  [N*K/64]          8-bit double-quantised block absmax
 *   dq_step [ceil(N*K/16384)] fp32 step of each group of 256 block scales
 *   dq_mean NULL for the unsigned scale format; otherwise [1] fp32, the
 *           tensor mean of the mean-centred format (qlora_double_quant_centred;
 *           4-byte aligned, EALIGN).
 * Block b covers flattened elements [64b, 64b+64) and decodes with scale
 *   unsigned:     s'_b = fp32(qscale[b] * dq_step[b/256])
 *   mean-centred: s'_b = fp32(fp32(int8(qscale[b]) * dq_step[b/256]) + dq_mean[0])
 * (int8: the byte read as two's complement; the product and the sum are
 * rounded separately).  Every call that takes a qlora_nf4_weight decodes
 * either format.                                                           */
typedef struct qlora_nf4_weight {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float*   dq_step;
  int64_t        N;
  int64_t        K;
  const float*   dq_mean;
} qlora_nf4_weight;

/* Blockwise NF4 quantisation.  [QLoRA / infivelines.com]: 16 levels at
 * normal quantiles; each block of 64 weights carries its own scale.
 *   w       [n_elems] fp32 input, flattened row-major (an [N, K] weight).
 *   codes   [ceil(n_elems/2)] packed 4-bit codes, even element in the low
 *           nibble; an odd tail is padded with code 7 (the zero level).
 *   absmax  [ceil(n_elems/64)] fp32 exact max |w| of each block (the last
 *           block may be partial).
 * A code is the index of the NF4 level nearest to fp32(w / absmax) (IEEE
 * correctly rounded quotient), ties to the lower level; a block whose
 * absmax is 0 gets code 7 everywhere.  blocksize must be 64 (ENOTSUP).
 * n_elems may be 0 (nothing is enqueued).                                   */
int qlora_quantize_nf4(const float* w, int64_t n_elems, int32_t blocksize,
                       uint8_t* codes, float* absmax, void* stream);

/* Double quantisation of block scales.  [QLoRA / infivelines.com]: the
 * block scales are quantised again in blocks of 256; [QLoRA -- Module 12.4,
 * "Double quant"]: quantise the quantisation constants.
 *   absmax  [n_blocks] fp32 block scales (>= 0), e.g. from the quantiser.
 *   qscale  [n_blocks] uint8: q = min(255, rint(fp32(absmax / step))).
 *   dq_step [ceil(n_blocks/256)] fp32: step = fp32(group max / 255);
 *           a group whose step is 0 stores q = 0.
 * Divisions are IEEE correctly rounded; rint is round-half-to-even.
 * blocksize2 must be 256 (ENOTSUP).                                         */
int qlora_double_quant(const float* absmax, int64_t n_blocks, int32_t blocksize2,
                       uint8_t* qscale, float* dq_step, void* stream);

/* Quantisation and double quantisation in one pass: the outputs of
 * qlora_quantize_nf4 (blocksize 64) followed by qlora_double_quant
 * (blocksize 256) on its absmax, bit for bit, from one read of w.
 * [QLoRA / infivelines.com]: NF4 blocks of 64, scales quantised again in
 * blocks of 256.  Arguments as in those two calls (absmax is still
 * written); n_elems may be 0 (nothing is enqueued); the five buffers must
 * not overlap (EINVAL) and must be 16-byte aligned (EALIGN).               */
int qlora_quantize_nf4_dq(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                          uint8_t* qscale, float* dq_step, void* stream);

/* Mean-centred double quantisation: the paper-style variant of the scale
 * format.  [QLoRA -- the democratization event, the recipe]: double
 * quantization as in the QLoRA paper the recipe cites, which centres the
 * block scales on their mean so that a symmetric 8-bit code can be used;
 * [QLoRA / infivelines.com]: groups of 256 scales.  The pages fix neither
 * this format nor the reduction order, so both are this library's reading:
 *   dq_mean [1] fp32: mu = fp32(T / n_blocks), T an fp64 sum -- each
 *           group's scales in index order, the group sums in 1024
 *           contiguous chunks of ceil(groups/1024) groups (in order), the
 *           chunk sums in chunk order (the same bits on every run);
 *   dq_step [ceil(n_blocks/256)] fp32: step = fp32(A / 127) with
 *           A = max |fp32(absmax - mu)| over the group's blocks;
 *   qscale  [n_blocks] two's-complement codes
 *           q = clamp(rint(fp32(fp32(absmax - mu) / step)), -127, 127);
 *           a group with A = 0 stores step 0 and q = 0.
 * Decoding (every call on a qlora_nf4_weight with dq_mean set):
 * s' = fp32(fp32(q * step) + mu).  Divisions are IEEE correctly rounded,
 * rint rounds half to even.  workspace (16-byte aligned) must hold
 * qlora_dq_centred_workspace_bytes(n_blocks) bytes (EWORKSPACE), no two
 * buffers may overlap (EINVAL); n_blocks may be 0 (nothing is enqueued).
 * Storage is that of the unsigned format plus the 4-byte mean.             */
size_t qlora_dq_centred_workspace_bytes(int64_t n_blocks);
int qlora_double_quant_centred(const float* absmax, int64_t n_blocks, uint8_t* qscale,
                               float* dq_step, float* dq_mean, void* workspace, size_t ws_bytes,
                               void* stream);
/* qlora_quantize_nf4 (blocksize 64) followed by qlora_double_quant_centred
 * on its absmax (written), with the workspace of
 * qlora_dq_centred_workspace_bytes(ceil(n_elems/64)).                       */
int qlora_quantize_nf4_dq_centred(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                                  uint8_t* qscale, float* dq_step, float* dq_mean,
                                  void* workspace, size_t ws_bytes, void* stream);

/* Standalone dequantisation to bf16 (the same device function the GEMMs
 * use): out[i] = bf16_rne(fp32(L[code_i] * s'_b)), s'_b the block's decoded
 * scale in the weight's format (above).
 * [QLoRA / infivelines.com]: the base is dequantised to bf16.
 *   out  [N*K] bf16 (uint16_t patterns), row-major [N, K].
 * Requires N*K to be a multiple of 64.                                      */
int qlora_dequantize_nf4(const qlora_nf4_weight* w, uint16_t* out, void* stream);

/* Forward pass.  [QLoRA / infivelines.com]: dequantised to bf16 one block
 * at a time inside the matrix multiply; adapters in full precision.
 *   x  [M, K] bf16        A [r, K] bf16        B [N, r] bf16
 *   y  [M, N] bf16 output: y = x.deq(W)^T + (alpha/r).(x.A^T).B^T,
 *      accumulated in fp32 and rounded once to bf16 (nearest-even).
 * M >= 1 is arbitrary; N and K must be multiples of 64 (ESHAPE), the
 * packed codes (N*K/2 bytes) and x and y (M*K*2, M*N*2 bytes) at most
 * 2 GiB each, and A, B and the adapter products (2*r*K, 2*N*r and
 * 4*r*(M rounded up to 32) bytes) below 2 GiB (ESHAPE: the kernels use
 * 32-bit byte offsets); r is 0 or a multiple of 8 up to 256 (r = 0: base
 * only, A and B may be NULL).
 * workspace: device scratch of at least
 * qlora_linear_workspace_bytes(0, M, N, K, r) bytes, 256-byte aligned.      */
int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                     uint16_t* y, void* workspace, size_t ws_bytes, void* stream);

/* Backward pass through the frozen base.  [QLoRA -- the democratization
 * event, the recipe]: gradients flow through the frozen 4-bit base into the
 * adapters; the base gets no gradient.
 *   dy [M, N] bf16 upstream gradient; x, A, B as in the forward pass.
 *   dx [M, K] bf16 output (may be NULL to skip):
 *        dx = dy.deq(W) + (alpha/r).(dy.B).A
 *   dA [r, K] fp32 output:  dA = (alpha/r).(dy.B)^T.x
 *   dB [N, r] fp32 output:  dB = (alpha/r).dy^T.(x.A^T)
 *   accumulate != 0 adds the new dA/dB to the existing contents.
 * r = 0: only dx is produced (A, B, dA, dB may be NULL).
 * Shapes and size limits as for the forward pass (ESHAPE).
 * workspace: at least qlora_linear_workspace_bytes(1, M, N, K, r) bytes.    */
int qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                     int64_t M, const uint16_t* A, const uint16_t* B, int32_t r,
                     float alpha, uint16_t* dx, float* dA, float* dB,
                     int32_t accumulate, void* workspace, size_t ws_bytes,
                     void* stream);

/* Merge the adapter into a base weight for export:
 *     W_m = W_base + (alpha/r) . B . A          ([N, K], row-major)
 * [QLoRA -- the democratization event, deployment note]: a merged model is
 * made by dequantising the base, merging the adapter, and possibly
 * quantising again.  [QLoRA / infivelines.com, the recipe's last step]:
 * merging into the 4-bit base and saving it loses precision twice; merge
 * against the original weights.  [QLoRA, and fine-tuning a 7B model on a
 * free GPU, "Merging a QLoRA adapter"]: merging into the full-precision
 * base is the usual practice.
 *   Base: exactly one of
 *     w   the NF4 weight, decoded exactly as qlora_dequantize_nf4 does
 *         (w->N == N and w->K == K), or
 *     w0  [N, K] fp32 original weights (e.g. the quantiser's input).
 *   A [r, K] bf16, B [N, r] bf16; r is 0 or a multiple of 8 up to 256
 *     (r = 0: W_m = W_base, A and B may be NULL).
 *   out_f32  [N, K] fp32:  fl32(W_base + s.U), one rounding, where U is the
 *            fp32 sum of the exact products B[n][j] * A[j][k] and
 *            s = fp32(alpha / r); may be NULL.
 *   out_bf16 [N, K] bf16:  that fp32 value rounded to nearest even; may be
 *            NULL.  At least one output must be given (EINVAL).
 *   To quantise the merge again, pass out_f32 to qlora_quantize_nf4_dq.
 * N and K must be multiples of 64 and N * r * 2 < 2^31 (ESHAPE).  Device
 * pointers, 16-byte aligned (EALIGN); outputs must not overlap each other
 * or the inputs (EINVAL).  No workspace.                                   */
int qlora_merge_adapter(const qlora_nf4_weight* w, const float* w0, int64_t N, int64_t K,
                        const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                        float* out_f32, uint16_t* out_bf16, void* stream);

/* The fp16 compute-type variant.  [QLoRA: Fine-Tuning a 7B Model on a 16GB
 * GPU, the flags paragraph]: compute_dtype float16 dequantises to fp16 for
 * the matrix multiplies.  The same layer and the same packed weight, with
 * every 16-bit tensor in IEEE binary16 instead of bf16:
 *   qlora_dequantize_nf4_f16: out[i] = fp16_rne(fp32(L[code_i] * s'_b))
 *   qlora_linear_fwd_f16 / qlora_linear_bwd_f16: x, A, B, y, dy, dx are
 *     fp16 (uint16_t patterns); dA, dB fp32; fp32 accumulation, y and dx
 *     rounded once to fp16 (nearest even).  Values beyond fp16's range
 *     overflow to infinity (not checked).
 * Arguments, errors and size limits as the bf16 calls; every M runs the
 * tiled GEMMs (no few-token path); workspace
 * qlora_linear_workspace_bytes(6 (forward) or 7 (backward), ...).         */
int qlora_dequantize_nf4_f16(const qlora_nf4_weight* w, uint16_t* out, void* stream);
int qlora_linear_fwd_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                         const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                         uint16_t* y, void* workspace, size_t ws_bytes, void* stream);
int qlora_linear_bwd_f16(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                         int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                         uint16_t* dx, float* dA, float* dB, int32_t accumulate, void* workspace,
                         size_t ws_bytes, void* stream);

/* Forward and backward with LoRA dropout on the adapter's input.
 * [QLoRA -- Module 12.4, "Hugging Face + BitsAndBytes"]: the adapter config
 * sets lora_dropout (0.05 there).  The pages give no formula; the standard
 * LoRA dropout is taken: the adapter sees x~ = x * keep / (1 - p), the base
 * term sees x, so
 *   y  = x.deq(W)^T + (alpha/r).(x~.A^T).B^T
 *   dx = dy.deq(W) + (alpha/r).((dy.B).A) * keep / (1 - p)
 *   dA = (alpha/r).(dy.B)^T.x~          dB = (alpha/r).dy^T.(x~.A^T)
 * The random draws are an input:
 *   keep [M, K/8] bytes (device, 16-byte aligned): bit (k mod 8) of byte
 *        (m, k/8) is 1 where x[m][k] is kept; the same mask must be passed
 *        to the backward of the same step.
 *   p    dropout probability, 0 <= p < 1 (EINVAL otherwise); 1/(1 - p) is
 *        folded into the fp32 scale alpha/r.
 * Other arguments, rounding (y and dx still rounded once), errors and size
 * limits as qlora_linear_fwd / qlora_linear_bwd; keep must not overlap an
 * output (EINVAL).  The forward takes the same paths as qlora_linear_fwd
 * (the few-token one for M <= 32); its workspace is
 * qlora_linear_workspace_bytes(4, ...), the backward's
 * qlora_linear_workspace_bytes(5, ...).  With r = 0 there is no adapter and
 * keep is ignored.                                                         */
int qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             const uint8_t* keep, float p, uint16_t* y, void* workspace,
                             size_t ws_bytes, void* stream);
int qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r,
                             float alpha, const uint8_t* keep, float p, uint16_t* dx, float* dA,
                             float* dB, int32_t accumulate, void* workspace, size_t ws_bytes,
                             void* stream);

/* LoRA dropout with the keep bits drawn by the library, from a
 * counter-based generator, instead of passed in.  [QLoRA -- Module 12.4,
 * "Hugging Face + BitsAndBytes"] sets lora_dropout (0.05); the generator
 * is Philox4x32 with ten rounds (Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC 2011).
 *   The keep bits of elements 8c .. 8c+7 of the flattened [M, K] x (mask
 *   byte c = m*(K/8) + k/8) come from one Philox call with counter
 *   (c, 0, offset lo, offset hi) and key (seed lo, seed hi): element 8c+j
 *   takes the 16-bit half j%2 (low first) of output word j/2, u, and is
 *   kept iff u >= t, t = nearest integer to 65536*p (ties to even).  The
 *   realised dropout probability is t/65536 (0.05 -> 0.0500031), and the
 *   inverted scaling uses it: the adapter sees x~ = x*keep/(1 - t/65536).
 *   The same (seed, offset) in the forward and the backward of a step
 *   draws the same bits (the backward draws them again; nothing is stored
 *   between the calls); use a new offset (or seed) for every step and
 *   layer.  0 <= p < 1 (EINVAL otherwise).
 *   qlora_dropout_keep_mask writes the bits the layer draws, in the
 *     packed layout of qlora_linear_fwd_dropout's keep argument ([M, K/8]
 *     bytes, 16-byte aligned; K a multiple of 8 and M*K*2 at most 2 GiB,
 *     ESHAPE), so qlora_linear_fwd_dropout with that mask and p =
 *     t/65536 computes the same layer.
 *   qlora_linear_fwd_dropout_rng / qlora_linear_bwd_dropout_rng: the
 *     layer of qlora_linear_fwd_dropout / qlora_linear_bwd_dropout with
 *     the drawn bits; other arguments, rounding, errors and size limits
 *     alike; the forward takes qlora_linear_fwd's paths; workspace
 *     qlora_linear_workspace_bytes(8 (forward) or 9 (backward), ...); the
 *     backward keeps the drawn mask in its workspace.                     */
int qlora_dropout_keep_mask(int64_t M, int64_t K, float p, uint64_t seed, uint64_t offset,
                            uint8_t* keep, void* stream);
int qlora_linear_fwd_dropout_rng(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                                 const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                                 float p, uint64_t seed, uint64_t offset, uint16_t* y,
                                 void* workspace, size_t ws_bytes, void* stream);
int qlora_linear_bwd_dropout_rng(const qlora_nf4_weight* w, const uint16_t* x,
                                 const uint16_t* dy, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float alpha, float p,
                                 uint64_t seed, uint64_t offset, uint16_t* dx, float* dA,
                                 float* dB, int32_t accumulate, void* workspace, size_t ws_bytes,
                                 void* stream);

/* The same layer with an unquantised bf16 base weight W [N, K] (row-major,
 * out x in), through the same kernels with the dequantisation left out:
 * the "LoRA on a 16-bit base" that QLoRA is compared with.
 * [QLoRA / infivelines.com]: because the base is dequantised on every
 * pass, training takes about a third longer than LoRA on an unquantised
 * base; [QLoRA, and fine-tuning a 7B model on a free GPU, "What it costs
 * in quality"]: where the bf16 model fits, bf16 training is the faster.
 *   y  = x.W^T + (alpha/r).(x.A^T).B^T                     (forward)
 *   dx = dy.W + (alpha/r).(dy.B).A,  dA, dB as in qlora_linear_bwd
 * Arguments, shapes (N, K multiples of 64), rounding, accumulation, errors
 * and size limits are those of qlora_linear_fwd / qlora_linear_bwd with
 * W in place of the packed weight (W 16-byte aligned, EALIGN).  Every M
 * runs the tiled GEMMs (there is no few-token path for this weight).
 * workspace: qlora_linear_workspace_bytes(2 (forward) or 3 (backward), ...). */
int qlora_linear_bf16_fwd(const uint16_t* W, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                          const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                          uint16_t* y, void* workspace, size_t ws_bytes, void* stream);
int qlora_linear_bf16_bwd(const uint16_t* W, int64_t N, int64_t K, const uint16_t* x,
                          const uint16_t* dy, int64_t M, const uint16_t* A, const uint16_t* B,
                          int32_t r, float alpha, uint16_t* dx, float* dA, float* dB,
                          int32_t accumulate, void* workspace, size_t ws_bytes, void* stream);

/* The forward pass of qlora_linear_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, kernels and
 * bits, with the workspace taken from a static device buffer that the
 * library holds instead of a caller argument.
 *   - The buffer is QLORA_NOALLOC_SCRATCH_BYTES (96 MiB) per GPU, allocated
 *     when the library's code is loaded on that GPU and held until the
 *     process ends.  A call whose workspace need,
 *     qlora_linear_workspace_bytes(0, M, N, K, r), exceeds it returns
 *     QLORA_ESCRATCH before any HIP call (every workload of this library
 *     fits: the largest, 2048 tokens through an 11008 -> 4096 layer, needs
 *     66.25 MiB).
 *   - The call allocates nothing (no hipMalloc, no hipFree).  On the first
 *     call on a GPU it looks up that GPU's copy of the buffer (a
 *     hipGetSymbolAddress with the current device, which must be the
 *     stream's device) and keeps the address.
 *   - Every call on one GPU shares that GPU's buffer: calls that may
 *     overlap in time on one GPU (different streams, or several host
 *     threads) race and give wrong results; serialise them (one stream) or
 *     use qlora_linear_fwd with separate workspaces.  The buffer keeps the
 *     last call's contents; no kernel reads what an earlier call left.
 * Arguments, shapes, rounding and other errors as qlora_linear_fwd.        */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             uint16_t* y, void* stream);

/* Workspace bytes for op 0 (forward) or 1 (backward) of the NF4 layer,
 * op 2 (forward) or 3 (backward) of the bf16-weight layer, op 4 (forward)
 * or 5 (backward) of the NF4 layer with dropout, op 6 (forward) or 7
 * (backward) of the fp16 compute type, or op 8 (forward) or 9 (backward)
 * of the NF4 layer with dropout drawn by the library, at the given shape;
 * 0 for an invalid shape.  Host-only; never touches the GPU.               */
size_t qlora_linear_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K,
                                    int32_t r);

/* The library's own fp32 NF4 table: the 16 levels, ascending, built on the
 * host from the library's own normal quantile function ("QLoRA"
 * (infivelines.com): 16 levels at equal-probability quantiles of a normal,
 * normalised to [-1, 1]).  `out` is a HOST pointer to 16 floats.  Returns
 * QLORA_EINVAL for a NULL `out`.  Never touches the GPU.                    */
int qlora_nf4_levels(float out[16]);

/* The quantiser's 15 fp32 decision thresholds between consecutive levels of
 * that table: threshold i is the midpoint of levels i and i + 1 rounded
 * towards -infinity, and code(u) = #{i : u > threshold[i]} is the nearest
 * level with ties to the lower one.  `out` is a HOST pointer to 15 floats.  Returns
 * QLORA_EINVAL for a NULL `out`.  Never touches the GPU.                    */
int qlora_nf4_thresholds(float out[15]);

/* Static string for a status code (host only).                             */
const char* qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
