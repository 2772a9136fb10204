// Internal launchers (one per device kernel family).  Every launcher
// enqueues on the given stream and returns hipGetLastError(); shapes and
// pointers have been validated by the C ABI layer before any call here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

struct qlora_nf4_weight;

namespace qlora {

// api.cpp -- the forward pass whose workspace comes from src(need, &status)
// once every argument has been validated (null with *status set on failure)
using WorkspaceSource = void* (*)(size_t need, int* status);
int linear_fwd_sourced(const qlora_nf4_weight* w, const uint16_t* x, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float alpha, uint16_t* y,
                       WorkspaceSource src, void* stream);

// quant_kernels.hip
hipError_t launch_quantize(const float* w, int64_t n, uint8_t* codes, float* absmax,
                           const Nf4CodeBins& bins, hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* qscale,
                               float* step, hipStream_t s);
// both in one pass (one workgroup per group of 256 blocks)
hipError_t launch_quantize_dq(const float* w, int64_t n, uint8_t* codes, float* absmax,
                              uint8_t* qscale, float* step, const Nf4CodeBins& bins,
                              hipStream_t s);
// the mean-centred scale format: mean [1], step [groups], qscale (signed
// codes) from the block scales; workspace of dq_centred_workspace_bytes
size_t dq_centred_workspace_bytes(int64_t nb);
hipError_t launch_double_quant_centred(const float* absmax, int64_t nb, uint8_t* qscale,
                                       float* step, float* mean, void* workspace,
                                       hipStream_t s);
// out: bf16, or fp16 (f16) -- the same decode rounded to the compute type
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const float* dq_mean, int64_t nb, uint16_t* out, const Nf4Levels& L,
                          hipStream_t s, bool f16 = false);

// lora_kernels.hip -- rank-r kernels of the adapter path
// lora_proj: out[m][j] = hi, out[m][r + j] = lo, the bf16 pair of
// v = scale * sum_k X[m][k] * Y(j, k), with Y(j, k) = Y[j * Kred + k]
// (kmajor == 0, A [r, Kred]) or Y[k * r + j] (kmajor == 1, B [Kred, r]);
// also outT[j][m] = hi, outT[r + j][m] = lo with rows of Mp = M rounded up
// to 32 (zero past M).  Each block reduces its whole range itself.
struct LoraProjJob {
  const uint16_t* X;  // [M, Kred] bf16
  const uint16_t* Y;
  uint16_t* out;      // [M, 2r] bf16
  uint16_t* outT;     // [2r, Mp] bf16
  int64_t Kred;
  int kmajor;
  // LoRA dropout on X (or null): [M, Kred / 8] bytes, bit k mod 8 of byte
  // (m, k / 8) set where X[m][k] is kept; dropped values count as zero
  const uint8_t* keep = nullptr;
  // LoRA dropout drawn in the kernel instead (rng != 0): the keep byte of
  // chunk (m, k / 8) is philox_keep_byte(drop, m Kred / 8 + k / 8); where
  // keep_out is given, the drawn bytes are also stored there ([M, Kred / 8])
  int rng = 0;
  PhiloxDrop drop{};
  uint8_t* keep_out = nullptr;
  // reduction split (lora_proj_plan): S > 1 blocks per (token, rank)
  // tile each sum a share of Kred into fp32 partials part [S][r][Mp], which
  // a finalize pass adds in split order
  int S = 1;
  float* part = nullptr;
};
// How lora_proj runs one or two jobs (reduction lengths kred0, kred1; 0 =
// no second job): the small kernel, or the MFMA kernel with TT 16-token
// tiles per block and S[j] reduction splits for job j.
struct ProjPlan {
  bool small;
  int tt;
  int s[2];
};
ProjPlan lora_proj_plan(int64_t M, int r, int64_t kred0, int64_t kred1);
// fp32 partials a job of the plan needs (0 when it is not split)
size_t lora_proj_partial_bytes(const ProjPlan& p, int job, int64_t M, int r);
// one job, or two in one launch (j1 non-null)
// f16: the fp16 compute type (operands and the hi/lo pairs in fp16; no
// keep-mask), else bf16.
// the packed keep mask [M, K / 8] that `drop` draws (philox_keep_byte)
hipError_t launch_dropout_mask(const PhiloxDrop& drop, int64_t M, int64_t K, uint8_t* keep,
                               hipStream_t s);
hipError_t launch_lora_proj(const LoraProjJob& j0, const LoraProjJob* j1, int64_t M, int r,
                            float scale, hipStream_t s, bool f16 = false);
// lora_grad: C (+)= sum_m G[m][g] * (ST[j][m] + ST[r + j][m]), C [ldg, r]
// (transposed == 0) or [r, ldg] (transposed == 1); both jobs in one launch,
// each block reducing over all tokens itself.
struct LoraGradJob {
  const uint16_t* G;   // [M, ldg] bf16, ldg a multiple of 64
  const uint16_t* ST;  // [2r, Mp] bf16 (hi rows, then lo rows), zero past M
  float* C;
  int64_t ldg;
  int transposed;
  const uint8_t* keep = nullptr;  // dropout mask on G, as in LoraProjJob (or null)
};
hipError_t launch_lora_grad(const LoraGradJob& j0, const LoraGradJob& j1, int64_t M, int r,
                            int accumulate, hipStream_t s, bool f16 = false);

// gemm_fwd.hip -- y = x . deq(W)^T + xs . [B | B]^T.
// Schedule of a fused GEMM with an Mout x Nout output (Nout in tiles of tn)
// and a reduction of Kred (in tiles of 64): either every tile's reduction is
// split `splits` ways (fp32 partials part[splits][M][Nout], reduced by
// splitk_reduce), or -- when the tiles fill at least one round of the chip
// -- the `full` first tiles run whole and the last tail_q tiles are split
// tail_s ways into tile-local fp32 partials tpart[tail_s][tail_q][tm][256],
// reduced by tail_reduce.
struct GemmConfig {
  int tm;        // token rows of the block tile (256 or 128)
  int splits;    // uniform reduction splits (1: none)
  int64_t full;  // tail schedule: tiles run whole
  int tail_q;    // tail schedule: split tiles (0: uniform schedule)
  int tail_s;    // tail schedule: splits per tail tile
  int tn;        // Nout extent of the block tile: 256, or 128 (the narrow
                 // 128 x 128 tile; never with the tail schedule)
};
// narrow: the 128 x 128 tile may be chosen (a GEMM on the NF4 weight)
GemmConfig gemm_config(int64_t M, int64_t Nout, int64_t Kred, bool narrow = false);
int64_t gemm_blocks(const GemmConfig& c, int64_t M, int64_t Nout);
size_t gemm_partial_bytes(const GemmConfig& c, int64_t M, int64_t Nout);
// The weight is the NF4 one (codes, qscale, step) when wbf is null, else the
// bf16 weight wbf [N, K] (the unquantised layer, same kernel skeleton).
// f16: the fp16 compute type (x, xs, B, y in fp16; the NF4 weight decoded
// to fp16); only with the NF4 weight.
// kWeightNf4Centred: the NF4 weight with the mean-centred scale format
// (dq_mean non-null); the same kernels, with that format's scale decode.
constexpr int kWeightNf4 = 0, kWeightBf16 = 1, kWeightNf4Centred = 2;
hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const float* dq_mean, const uint16_t* wbf, const uint16_t* x,
                           const uint16_t* xs, const uint16_t* B, uint16_t* y, float* part,
                           int64_t M, int64_t N,
                           int64_t K, int r, const Nf4Levels& L, hipStream_t s,
                           bool f16 = false);
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                                hipStream_t s, bool f16 = false);
// the reduction after a fused GEMM's main kernel, if its schedule has one
hipError_t launch_gemm_reduce(const GemmConfig& c, const float* part, int64_t M, int64_t Nout,
                              uint16_t* out, hipStream_t s, bool f16 = false);

// gemm_decode.hip -- forward for M <= 32.  Without an adapter one kernel
// writes y.  With one, a first launch of k-split A tiles writes the
// partials of x . A^T to part[z][m][j] ([S][M][r] fp32), then the weight
// tiles write y = bf16(x . W'^T + scale . (sum_z part[z]) . B^T);
// decode_splits is the number of partial planes S (0: none).  keep or drop
// (or neither): LoRA dropout on the adapter's input, as in lora_proj.
constexpr int kDecodeMaxM = 32;
int decode_splits(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* qscale, const float* step,
                             const float* dq_mean, const uint16_t* x, const uint16_t* A,
                             const uint16_t* B, int r,
                             float scale, float* part, int splits, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, const Nf4Levels& L, hipStream_t s,
                             const uint8_t* keep = nullptr, const PhiloxDrop* drop = nullptr);

// gemm_bwd.hip -- dx = dy . deq(W) + gs . [A ; A]; scheduled by
// gemm_config(M, K, N) (output M x K, reduction N)
// keep (or null): LoRA dropout bits [M, K / 8] masking the adapter term.
hipError_t launch_dx_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const float* dq_mean, const uint16_t* wbf, const uint8_t* keep,
                          const uint16_t* dy,
                          const uint16_t* gs, const uint16_t* A, uint16_t* dx, float* part,
                          int64_t M, int64_t N, int64_t K, int r, const Nf4Levels& L,
                          hipStream_t s, bool f16 = false);

// merge.hip -- W_m = W_base + scale . B . A for export.  The base is the NF4
// weight (codes non-null) or the fp32 original w0; out_f32 and/or out_bf16
// [N, K]; N, K multiples of 64, N * r * 2 < 2^31.  One wave per 64-column
// strip of K and `tiles_per_wave` 32-row tiles of N.
constexpr int64_t kMergeTargetWaves = 4096;
struct MergePlan {
  int tiles_per_wave;
  int64_t waves;
  int64_t blocks;  // 4 waves each
};
MergePlan merge_plan(int64_t N, int64_t K);
hipError_t launch_merge(const uint8_t* codes, const uint8_t* qscale, const float* step,
                        const float* dq_mean, const float* w0, const uint16_t* A,
                        const uint16_t* B, int r,
                        float scale, float* out_f32, uint16_t* out_bf16, int64_t N, int64_t K,
                        const Nf4Levels& L, hipStream_t s);

}  // namespace qlora
