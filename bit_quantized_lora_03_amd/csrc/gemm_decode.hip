// Forward pass for few tokens (M <= 32): the decode-shaped, HBM-bound case.
//
// [QLoRA / infivelines.com]: the base is stored in 4 bits and dequantised to
// bf16 one block at a time inside the matrix multiply.  With a handful of
// tokens each decoded weight is used only M times, so the pass is a stream
// over the packed weight (~4.13 bits per weight) and the work per weight is
// the decode itself.  Here every weight is decoded exactly once, straight
// into MFMA operand registers (no LDS round trip):
//
//  * a 32x32x16 MFMA takes 32 weight rows (n) as its A operand and the
//    (zero-padded) tokens as its 32 B columns;
//  * lane (row l%32, half l/32) owns one whole 64-weight block per 128-wide
//    k span, so it builds that block's 16-entry table once and decodes its
//    64 codes into the A operands of 8 consecutive MFMAs.  The reduction
//    order over k is permuted consistently for A and B (MFMA j of a span
//    sums k = base + 64 g + 8 j + e over g = 0, 1 and e = 0..7);
//  * each x operand is loaded once per span and reused for the 4 row
//    subtiles of the wave.
//
// Grid: (ceil(N / 128) row tiles) x S k-splits; 4 waves per block split the
// block's k range again.  Partial sums go to an fp32 workspace
// part[S][M][N]; decode_reduce adds them in a fixed order, adds the adapter
// term (alpha/r) . (x . A^T) . B^T in fp32 and rounds to bf16 once.

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int ROWS = 128;       // weight rows per block
constexpr int SUB = 4;          // 32-row MFMA subtiles per wave
constexpr int SPAN = 128;       // k per span (two 64-weight blocks per row)

struct DecodeParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* x;
  float* part;
  int64_t M, N, K;
  int64_t spans_per_wave;
  Nf4Levels L;
};

}  // namespace

__global__ __launch_bounds__(256) void decode_main_kernel(DecodeParams p) {
  __shared__ float red[4][ROWS][33];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int z = blockIdx.y;
  const int64_t M = p.M, N = p.N, K = p.K;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  f32x16_t acc[SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  const int64_t spans_total = (K + SPAN - 1) / SPAN;
  const int64_t s_begin = ((int64_t)z * 4 + wave) * p.spans_per_wave;
  const int64_t s_end = s_begin + p.spans_per_wave < spans_total ? s_begin + p.spans_per_wave
                                                                 : spans_total;
  const bool tok_ok = lr < M;

  for (int64_t sp = s_begin; sp < s_end; ++sp) {
    const int64_t kb = sp * SPAN + 64 * lg;  // this lane's block start along k
    const bool kb_ok = kb < K;
    // x operands for the 8 MFMAs of the span (token lr, k = kb + 8j .. +8)
    u32x4_t xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      xb[j] = (tok_ok && kb_ok) ? *reinterpret_cast<const u32x4_t*>(p.x + lr * K + kb + 8 * j)
                                : zero;
    // codes and scales of the lane's block in each subtile row
    u32x4_t cr[SUB][2];
    float sc[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const int64_t n = n0 + 32 * i + lr;
      if (n < N && kb_ok) {
        const int64_t idx = n * K + kb;
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(p.codes + (idx >> 1));
        cr[i][0] = cp[0];
        cr[i][1] = cp[1];
        sc[i] = nf4_block_scale(p.qscale[idx >> 6], p.step[idx >> 14]);
      } else {
        cr[i][0] = zero;
        cr[i][1] = zero;
        sc[i] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const Nf4Lut lut = nf4_make_lut(p.L, sc[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i] = mfma32x32x16(nf4_decode8(lut, cr[i][j >> 2][j & 3]), xb[j], acc[i]);
    }
  }

  // D[n][m]: lane holds token m = lr, rows n = 8(v/4) + 4 lg + v%4
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      red[wave][32 * i + 8 * (v >> 2) + 4 * lg + (v & 3)][lr] = acc[i][v];
  __syncthreads();
  for (int e = t; e < ROWS * 32; e += 256) {
    const int row = e >> 5, m = e & 31;
    const int64_t n = n0 + row;
    if (m < M && n < N) {
      const float s = red[0][row][m] + red[1][row][m] + red[2][row][m] + red[3][row][m];
      p.part[((int64_t)z * M + m) * N + n] = s;
    }
  }
}

// y[m][n] = bf16( sum_z part[z][m][n] + scale * sum_j xa[m][j] B[n][j] ),
// xa[m][j] = sum_z' P[z'][m][j] (fixed summation orders).  One thread per
// output column n; its B row is read once, 8 values at a time.
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ P, int psplits,
    const uint16_t* __restrict__ B, int r, float scale, uint16_t* __restrict__ y, int64_t M,
    int64_t N) {
  __shared__ float xa[32 * 256];
  const int t = threadIdx.x;
  for (int e = t; e < M * r; e += 256) {
    float s = 0.0f;
    for (int z = 0; z < psplits; ++z) s += P[(int64_t)z * M * r + e];
    xa[e] = s;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 256 + t;
  if (n >= N) return;
  float lsum[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) lsum[m] = 0.0f;
  for (int jc = 0; jc < r; jc += 8) {
    const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(B + n * r + jc);
    float b[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[2 * e] = bf16_bits_to_f32(bv[e] & 0xFFFFu);
      b[2 * e + 1] = bf16_bits_to_f32(bv[e] >> 16);
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if (m < M) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum[m] += xa[m * r + jc + e] * b[e];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    if (m < M) {
      float acc = 0.0f;
      for (int z = 0; z < splits; ++z) acc += part[((int64_t)z * M + m) * N + n];
      acc += scale * lsum[m];
      y[m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
  }
}

int decode_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + ROWS - 1) / ROWS;
  const int64_t spans = (K + SPAN - 1) / SPAN;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t cap = spans / 4 > 0 ? spans / 4 : 1;  // every wave gets >= 1 span
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* qscale, const float* step,
                             const uint16_t* x, const float* P, int psplits, const uint16_t* B,
                             int r, float scale, float* part, int splits, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, const Nf4Levels& L, hipStream_t s) {
  DecodeParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.x = x;
  p.part = part;
  p.M = M;
  p.N = N;
  p.K = K;
  const int64_t spans = (K + SPAN - 1) / SPAN;
  p.spans_per_wave = (spans + 4 * splits - 1) / (4 * splits);
  p.L = L;
  dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)splits);
  hipLaunchKernelGGL(decode_main_kernel, grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                     part, splits, P, psplits, B, r, scale, y, M, N);
  return hipGetLastError();
}

}  // namespace qlora
