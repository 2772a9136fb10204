// Internal launchers (one per device kernel family).  Every launcher
// enqueues on the given stream and returns hipGetLastError(); shapes and
// pointers have been validated by the C ABI layer before any call here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace qlora {

// quant_kernels.hip
hipError_t launch_quantize(const float* w, int64_t n, uint8_t* codes, float* absmax,
                           const Nf4Thresholds& T, hipStream_t s);
hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* qscale,
                               float* step, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          int64_t nb, uint16_t* out, const Nf4Levels& L, hipStream_t s);

// lora_kernels.hip -- rank-r helper GEMMs
// Partial products P[z][m][j] = sum over the z-th share of the k range of
// X[m][k] * Y[j][k]; X [M, K] and Y [R, K] bf16 row-major.
int lora_down_splits(int64_t M, int64_t K, int R);
hipError_t launch_lora_down(const uint16_t* X, const uint16_t* Y, int64_t M, int64_t K, int R,
                            int splits, float* P, hipStream_t s);
// out[m][c], c in [0, 2R): hi / lo bf16 split of v = scale * sum_z P[z][m][c mod R]
hipError_t launch_lora_split(const float* P, int splits, int64_t M, int R, float scale,
                             uint16_t* out, hipStream_t s);
// dst [C, R] = transpose of src [R, C] (bf16)
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t s);
// C[p][q] (+)= sum_h sum_m U_h[m][p] * V_h[m][q] for h in {0, 1}; U_h has
// leading dimension ldu, V_h ldv; C [P, Q] fp32 row-major.
hipError_t launch_tn_gemm(const uint16_t* U0, const uint16_t* U1, int64_t ldu,
                          const uint16_t* V0, const uint16_t* V1, int64_t ldv, int64_t M,
                          int64_t P, int64_t Q, float* C, int accumulate, hipStream_t s);

// gemm_fwd.hip -- y = x . deq(W)^T + xs . [B | B]^T.  With splits > 1 the
// k range is split over blocks writing fp32 partials part[splits][M][N],
// reduced to bf16 y by a second kernel.
int gemm_splits(int64_t M, int64_t N, int64_t Kred);
hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const uint16_t* x, const uint16_t* xs, const uint16_t* B,
                           uint16_t* y, float* part, int splits, int64_t M, int64_t N, int64_t K,
                           int r, const Nf4Levels& L, hipStream_t s);
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                                hipStream_t s);

// gemm_decode.hip -- forward for M <= 32: split-K partials
// part[S][M][N + r] (columns N.. hold x . A^T), then
// y = bf16(sum part + scale . xa . B^T)
constexpr int kDecodeMaxM = 32;
int decode_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* qscale, const float* step,
                             const uint16_t* x, const uint16_t* A, const uint16_t* B, int r,
                             float scale, float* part, int splits, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, const Nf4Levels& L, hipStream_t s);

// gemm_bwd.hip -- dx = dy . deq(W) + gs . [A ; A]; splits > 1 as in the
// forward GEMM (partials [splits][M][K])
hipError_t launch_dx_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const uint16_t* dy, const uint16_t* gs, const uint16_t* A,
                          uint16_t* dx, float* part, int splits, int64_t M, int64_t N, int64_t K,
                          int r, const Nf4Levels& L, hipStream_t s);

}  // namespace qlora
