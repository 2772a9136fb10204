// Rank-r helper GEMMs of the LoRA path (gfx950, bf16 MFMA, fp32 accumulate).
//
// The adapter path y += s . (x . A^T) . B^T and its gradients are skinny
// GEMMs with one dimension equal to the rank r ("QLoRA -- Module 12.4",
// "Hugging Face + BitsAndBytes": LoraConfig(r, lora_alpha); s = alpha / r).
//
//  * lora_down: P[z] = X . Y^T over the z-th share of the reduction, for
//    x . A^T (forward) and dy . B (backward, with B transposed first).  The
//    reduction is long (K or N) and the output thin, so the work is split
//    over the reduction into fp32 partials summed later in a fixed order.
//  * lora_split: v = s . sum_z P[z] rounded to a bf16 pair (hi, lo) with
//    hi + lo = v to 2^-17 relative, so that the rank-r product can ride on
//    bf16 MFMA in the big GEMMs' epilogues without losing the fp32 value.
//  * tn_gemm: dB = dy^T . xs and dA = gs^T . x, reductions over the tokens.

#include "device_common.h"
#include "launch.h"

namespace qlora {

// ---------------------------------------------------------------------------
// lora_down: grid (ceil(M/64), splits, ceil(R/64)), 256 threads.  Each wave
// takes every 4th 64-wide k tile of the block's share and computes a 64x64
// (m x j) tile with 32x32x16 MFMA straight from global memory (X rows and
// Y rows are both k-contiguous).  The four waves' tiles are summed in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ Y,
                                                        int64_t M, int64_t K, int R, int splits,
                                                        float* __restrict__ P) {
  __shared__ float red[4][64][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int z = blockIdx.y;
  const int j0 = blockIdx.z * 64;
  const int64_t nkt = K >> 6;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  for (int64_t kt = z + (int64_t)splits * wave; kt < nkt; kt += (int64_t)splits * 4) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t k = kt * 64 + kk * 16 + 8 * lg;
      u32x4_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t m = m0 + 32 * i + lr;
        a[i] = (m < M) ? *reinterpret_cast<const u32x4_t*>(X + m * K + k) : zero;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int jr = j0 + 32 * j + lr;
        b[j] = (jr < R) ? *reinterpret_cast<const u32x4_t*>(Y + (int64_t)jr * K + k) : zero;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  }
  // D = X . Y^T: lane holds column j = lr, rows m = 8(v/4) + 4 lg + v%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[wave][32 * i + 8 * (v >> 2) + 4 * lg + (v & 3)][32 * j + lr] = acc[i][j][v];
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int mm = e >> 6, jj = e & 63;
    const float s = red[0][mm][jj] + red[1][mm][jj] + red[2][mm][jj] + red[3][mm][jj];
    const int64_t m = m0 + mm;
    const int j = j0 + jj;
    if (m < M && j < R) P[((int64_t)z * M + m) * R + j] = s;
  }
}

int lora_down_splits(int64_t M, int64_t K, int R) {
  const int64_t mt = (M + 63) / 64, jt = (R + 63) / 64;
  const int64_t nkt = K / 64;
  int64_t cap = nkt / 4;
  if (cap < 1) cap = 1;
  int64_t s = (512 + mt * jt - 1) / (mt * jt);
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_lora_down(const uint16_t* X, const uint16_t* Y, int64_t M, int64_t K, int R,
                            int splits, float* P, hipStream_t s) {
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)splits, (unsigned)((R + 63) / 64));
  hipLaunchKernelGGL(lora_down_kernel, grid, dim3(256), 0, s, X, Y, M, K, R, splits, P);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_split: out[m][j] = hi, out[m][R + j] = lo with v = scale * sum_z P,
// hi = bf16(v), lo = bf16(v - hi) (v - hi is exact in fp32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_rne_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__global__ __launch_bounds__(256) void lora_split_kernel(const float* __restrict__ P, int splits,
                                                         int64_t M, int R, float scale,
                                                         uint16_t* __restrict__ out) {
  const int64_t total = M * R;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    float acc = 0.0f;
    for (int z = 0; z < splits; ++z) acc += P[(int64_t)z * total + e];
    const float v = scale * acc;
    const uint16_t hi = bf16_rne_bits(v);
    const uint16_t lo = bf16_rne_bits(v - bf16_bits_to_f32(hi));
    const int64_t m = e / R;
    const int j = (int)(e - m * R);
    out[m * 2 * R + j] = hi;
    out[m * 2 * R + R + j] = lo;
  }
}

hipError_t launch_lora_split(const float* P, int splits, int64_t M, int R, float scale,
                             uint16_t* out, hipStream_t s) {
  const int64_t total = M * R;
  int64_t g = (total + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(lora_split_kernel, dim3((unsigned)g), dim3(256), 0, s, P, splits, M, R,
                     scale, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// transpose (bf16): dst[c][r] = src[r][c], 64x64 tiles through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             int64_t R, int64_t C,
                                                             uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int rr = e >> 6, cc = e & 63;
    const int64_t r = r0 + rr, c = c0 + cc;
    tile[rr][cc] = (r < R && c < C) ? src[r * C + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int cc = e >> 6, rr = e & 63;
    const int64_t r = r0 + rr, c = c0 + cc;
    if (r < R && c < C) dst[c * R + r] = tile[rr][cc];
  }
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t s) {
  dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, src, R, C, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tn_gemm: C[p][q] (+)= sum_h sum_m U_h[m][p] V_h[m][q].  The reduction runs
// over the tokens m, the slow dimension of both operands, so each 64-token
// step is stored transposed in LDS (tokens contiguous) and read back as
// MFMA operands.  grid (ceil(P/64), ceil(Q/64)), 256 threads; wave (wp, wq)
// owns a 32x32 quadrant.  Each output tile is reduced by one block over all
// tokens, in a fixed order.
// ---------------------------------------------------------------------------
// LDS tile [64 rows][64 tokens] bf16, rows 128 B; 16-byte token chunks are
// swizzled by the row so that both the transposing 2-byte writes (8 rows
// at once) and the 16-byte operand reads (8 consecutive rows) spread over
// all banks.
__device__ __forceinline__ int tn_off(int row, int tok) {
  const int chunk = (tok >> 3) ^ (row & 7) ^ ((row >> 3) & 7);
  return row * 64 + chunk * 8 + (tok & 7);
}

__global__ __launch_bounds__(256) void tn_gemm_kernel(
    const uint16_t* __restrict__ U0, const uint16_t* __restrict__ U1, int64_t ldu,
    const uint16_t* __restrict__ V0, const uint16_t* __restrict__ V1, int64_t ldv, int64_t M,
    int64_t P, int64_t Q, float* __restrict__ C, int accumulate) {
  __shared__ uint16_t ut[2][64 * 64];
  __shared__ uint16_t vt[2][64 * 64];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wp = wave & 1, wq = wave >> 1;
  const int64_t p0 = (int64_t)blockIdx.x * 64, q0 = (int64_t)blockIdx.y * 64;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  const int chunk = t & 7;  // 8 columns (p or q) per thread per row
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* U = h ? U1 : U0;
      const uint16_t* V = h ? V1 : V0;
#pragma unroll
      for (int rep = 0; rep < 2; ++rep) {
        const int tok = (t >> 3) + 32 * rep;
        const int64_t m = m0 + tok;
        const int64_t p = p0 + 8 * chunk, q = q0 + 8 * chunk;
        const u32x4_t u = (m < M && p < P) ? *reinterpret_cast<const u32x4_t*>(U + m * ldu + p) : zero;
        const u32x4_t v = (m < M && q < Q) ? *reinterpret_cast<const u32x4_t*>(V + m * ldv + q) : zero;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t uw = u[e >> 1], vw = v[e >> 1];
          ut[h][tn_off(8 * chunk + e, tok)] = (uint16_t)((e & 1) ? (uw >> 16) : uw);
          vt[h][tn_off(8 * chunk + e, tok)] = (uint16_t)((e & 1) ? (vw >> 16) : vw);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int tc = 2 * kk + lg;  // token chunk
        const int pr = 32 * wp + lr, qr = 32 * wq + lr;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&ut[h][tn_off(pr, 8 * tc)]);
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&vt[h][tn_off(qr, 8 * tc)]);
        acc = mfma32x32x16(a, b, acc);
      }
    }
    __syncthreads();
  }
  // D[p][q]: lane holds column q = 32 wq + lr, rows p = 32 wp + 8(v/4) + 4 lg + v%4.
  const int64_t q = q0 + 32 * wq + lr;
  if (q < Q) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t p = p0 + 32 * wp + 8 * (v >> 2) + 4 * lg + (v & 3);
      if (p < P) {
        float* c = C + p * Q + q;
        *c = accumulate ? (*c + acc[v]) : acc[v];
      }
    }
  }
}

hipError_t launch_tn_gemm(const uint16_t* U0, const uint16_t* U1, int64_t ldu,
                          const uint16_t* V0, const uint16_t* V1, int64_t ldv, int64_t M,
                          int64_t P, int64_t Q, float* C, int accumulate, hipStream_t s) {
  dim3 grid((unsigned)((P + 63) / 64), (unsigned)((Q + 63) / 64));
  hipLaunchKernelGGL(tn_gemm_kernel, grid, dim3(256), 0, s, U0, U1, ldu, V0, V1, ldv, M, P, Q,
                     C, accumulate);
  return hipGetLastError();
}

}  // namespace qlora
