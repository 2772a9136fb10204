// Forward pass for few tokens (M <= 32): the decode-shaped, HBM-bound case.
//
// [QLoRA / infivelines.com]: the base is stored in 4 bits and dequantised to
// bf16 one block at a time inside the matrix multiply.  With a handful of
// tokens each decoded weight is used only M times, so the pass is a stream
// over the packed weight (~4.13 bits per weight) and the work per weight is
// the decode itself.  Every weight is decoded exactly once, straight into
// MFMA operand registers (no LDS round trip for weights):
//
//  * a 32x32x16 MFMA takes 32 weight rows (n) as its A operand and the
//    (zero-padded) tokens as its 32 B columns;
//  * lane (row l%32, half l/32) owns one whole 64-weight block per 128-wide
//    k span, so it builds that block's 16-entry table once and decodes its
//    64 codes into the A operands of 8 consecutive MFMAs.  The reduction
//    order over k is permuted consistently for A and B (MFMA j of a span
//    sums k = base + 64 g + 8 j + e over g = 0, 1 and e = 0..7);
//  * the block's slice of x sits in LDS (read once from global), and each x
//    operand read serves the 4 row subtiles of the wave;
//  * the next span's codes and scales are loaded while the current span is
//    decoded, so every wave keeps its weight bytes in flight.
//
// The adapter's down projection x . A^T rides along: rows N .. N+r-1 of the
// partial output are the rows of A (bf16, used as they are), so one pass
// produces both the base partial sums and the x . A^T partials.
//
// Grid: (ceil(N/128) + ceil(r/128) row tiles) x S k-splits; the 4 waves of a
// block split its k range again.  Partial sums go to part[S][M][N + r];
// decode_reduce adds them in a fixed order, forms the fp32 adapter term
// (alpha/r) . (x . A^T) . B^T and rounds y to bf16 once.

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int ROWS = 128;  // rows per block tile
constexpr int SUB = 4;     // 32-row MFMA subtiles per wave
constexpr int SPAN = 128;  // k per span (two 64-weight blocks per row)

struct DecodeParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* x;
  const uint16_t* A;
  float* part;
  int64_t M, N, K;
  int r;
  int64_t spans_per_wave;
  int64_t x_stride;  // LDS row stride of the x slice, in bf16 elements
  Nf4Levels L;
};

struct SpanRegs {
  u32x4_t c[SUB][2];
  float s[SUB];
};

}  // namespace

__global__ __launch_bounds__(256) void decode_main_kernel(DecodeParams p) {
  extern __shared__ u32x4_t dyn_lds[];
  uint16_t* xl = reinterpret_cast<uint16_t*>(dyn_lds);
  float* red = reinterpret_cast<float*>(dyn_lds);

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t ntiles = (N + ROWS - 1) / ROWS;
  const bool a_tile = blockIdx.x >= ntiles;  // rows of A instead of weight rows
  const int64_t n0 = (a_tile ? (int64_t)(blockIdx.x - ntiles) : (int64_t)blockIdx.x) * ROWS;
  const int64_t nrows = a_tile ? p.r : N;
  const int z = blockIdx.y;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  const int64_t spans_total = (K + SPAN - 1) / SPAN;
  const int64_t blk_span0 = (int64_t)z * 4 * p.spans_per_wave;
  int64_t blk_span1 = blk_span0 + 4 * p.spans_per_wave;
  if (blk_span1 > spans_total) blk_span1 = spans_total;
  const int64_t kx0 = blk_span0 * SPAN;                 // first k of the block's slice
  const int64_t kx1 = blk_span1 * SPAN < K ? blk_span1 * SPAN : K;

  // ---- stage the block's slice of x (M rows, [kx0, kx1)) into LDS ----
  {
    const int64_t chunks = (kx1 - kx0) >> 3;  // 8 bf16 per 16-byte chunk
    for (int64_t e = t; e < M * chunks; e += 256) {
      const int64_t m = e / chunks, c = e - m * chunks;
      *reinterpret_cast<u32x4_t*>(xl + m * p.x_stride + 8 * c) =
          *reinterpret_cast<const u32x4_t*>(p.x + m * K + kx0 + 8 * c);
    }
  }
  __syncthreads();

  f32x16_t acc[SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  const int64_t s_begin = blk_span0 + wave * p.spans_per_wave;
  const int64_t s_end = s_begin + p.spans_per_wave < blk_span1 ? s_begin + p.spans_per_wave
                                                               : blk_span1;
  const bool tok_ok = lr < M;

  auto load_span = [&](int64_t sp, SpanRegs& R) {
    const int64_t kb = sp * SPAN + 64 * lg;
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const int64_t n = n0 + 32 * i + lr;
      if (n < nrows && kb < K) {
        const int64_t idx = n * K + kb;
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(p.codes + (idx >> 1));
        R.c[i][0] = cp[0];
        R.c[i][1] = cp[1];
        R.s[i] = nf4_block_scale(p.qscale[idx >> 6], p.step[idx >> 14]);
      } else {
        R.c[i][0] = zero;
        R.c[i][1] = zero;
        R.s[i] = 0.0f;
      }
    }
  };
  auto x_operands = [&](int64_t sp, u32x4_t (&xb)[8]) {
    const int64_t kb = sp * SPAN + 64 * lg;
    const bool ok = tok_ok && kb < K;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      xb[j] = ok ? *reinterpret_cast<const u32x4_t*>(xl + lr * p.x_stride + (kb - kx0) + 8 * j)
                 : zero;
  };

  if (!a_tile) {
    SpanRegs cur, nxt;
    if (s_begin < s_end) load_span(s_begin, cur);
    for (int64_t sp = s_begin; sp < s_end; ++sp) {
      if (sp + 1 < s_end) load_span(sp + 1, nxt);
      u32x4_t xb[8];
      x_operands(sp, xb);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const Nf4Lut lut = nf4_make_lut(p.L, cur.s[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i] = mfma32x32x16(nf4_decode8(lut, cur.c[i][j >> 2][j & 3]), xb[j], acc[i]);
      }
      cur = nxt;
    }
  } else {
    // rows of A: bf16 operands as stored
    for (int64_t sp = s_begin; sp < s_end; ++sp) {
      const int64_t kb = sp * SPAN + 64 * lg;
      u32x4_t xb[8];
      x_operands(sp, xb);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int64_t j = n0 + 32 * i + lr;
        const bool ok = j < nrows && kb < K;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const u32x4_t av =
              ok ? *reinterpret_cast<const u32x4_t*>(p.A + j * K + kb + 8 * jj) : zero;
          acc[i] = mfma32x32x16(av, xb[jj], acc[i]);
        }
      }
    }
  }

  // ---- sum the 4 waves' partials in LDS (reusing the x slice's space) ----
  __syncthreads();
  const int mcols = (int)M;
  // D[n][m]: lane holds token m = lr, rows n = 8(v/4) + 4 lg + v%4
  if (tok_ok) {
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        red[(wave * ROWS + 32 * i + 8 * (v >> 2) + 4 * lg + (v & 3)) * mcols + lr] = acc[i][v];
  }
  __syncthreads();
  const int64_t col0 = a_tile ? N + n0 : n0;
  const int64_t ldp = N + p.r;
  for (int e = t; e < ROWS * mcols; e += 256) {
    const int row = e / mcols, m = e - row * mcols;
    if (n0 + row < nrows) {
      const float s = red[(0 * ROWS + row) * mcols + m] + red[(1 * ROWS + row) * mcols + m] +
                      red[(2 * ROWS + row) * mcols + m] + red[(3 * ROWS + row) * mcols + m];
      p.part[((int64_t)z * M + m) * ldp + col0 + row] = s;
    }
  }
}

// y[m][n] = bf16( sum_z part[z][m][n] + scale * sum_j xa[m][j] B[n][j] ) with
// xa[m][j] = sum_z part[z][m][N + j]; fixed summation orders.  Block of 256
// threads = 64 columns n x 4 token groups.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part,
                                                            int splits,
                                                            const uint16_t* __restrict__ B,
                                                            int r, float scale,
                                                            uint16_t* __restrict__ y, int64_t M,
                                                            int64_t N) {
  __shared__ float xa[32 * 256];
  const int t = threadIdx.x;
  const int64_t ldp = N + r;
  for (int e = t; e < M * r; e += 256) {
    const int64_t m = e / r, j = e - m * r;
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += part[((int64_t)z * M + m) * ldp + N + j];
    xa[e] = s;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 64 + (t & 63);
  const int mg = t >> 6;
  if (n >= N) return;
  constexpr int MPT = 8;  // tokens per thread (M <= 32, 4 groups)
  float lsum[MPT];
#pragma unroll
  for (int i = 0; i < MPT; ++i) lsum[i] = 0.0f;
  for (int jc = 0; jc < r; jc += 8) {
    const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(B + n * r + jc);
    float b[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[2 * e] = bf16_bits_to_f32(bv[e] & 0xFFFFu);
      b[2 * e + 1] = bf16_bits_to_f32(bv[e] >> 16);
    }
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const int m = mg + 4 * i;
      if (m < M) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum[i] += xa[m * r + jc + e] * b[e];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MPT; ++i) {
    const int m = mg + 4 * i;
    if (m < M) {
      float acc = 0.0f;
      for (int z = 0; z < splits; ++z) acc += part[((int64_t)z * M + m) * ldp + n];
      acc += scale * lsum[i];
      y[m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
  }
}

// Splits of k across blocks: enough blocks to fill the chip (~512), every
// wave at least one span, and the block's x slice (M rows of its k range)
// within 80 KiB of LDS so that two blocks fit on a CU.
int decode_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = (N + ROWS - 1) / ROWS;
  const int64_t spans = (K + SPAN - 1) / SPAN;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t cap = spans / 4 > 0 ? spans / 4 : 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  const int64_t mm = M > 0 ? M : 1;
  int64_t spw_max = ((80 * 1024) / (2 * mm) - 8) / (4 * SPAN);
  if (spw_max < 1) spw_max = 1;
  const int64_t s_min = (spans + 4 * spw_max - 1) / (4 * spw_max);
  if (s < s_min) s = s_min;
  return (int)s;
}

hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* qscale, const float* step,
                             const uint16_t* x, const uint16_t* A, const uint16_t* B, int r,
                             float scale, float* part, int splits, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, const Nf4Levels& L, hipStream_t s) {
  DecodeParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.x = x;
  p.A = A;
  p.part = part;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  const int64_t spans = (K + SPAN - 1) / SPAN;
  p.spans_per_wave = (spans + 4 * splits - 1) / (4 * splits);
  // x slice row stride: the block's k extent plus 8 (one 16-byte chunk of
  // padding staggers the rows across LDS banks)
  p.x_stride = 4 * p.spans_per_wave * SPAN + 8;
  p.L = L;
  const size_t x_bytes = (size_t)M * p.x_stride * sizeof(uint16_t);
  const size_t red_bytes = (size_t)4 * ROWS * M * sizeof(float);
  const size_t lds = x_bytes > red_bytes ? x_bytes : red_bytes;
  const unsigned tiles = (unsigned)((N + ROWS - 1) / ROWS + (r + ROWS - 1) / ROWS);
  hipLaunchKernelGGL(decode_main_kernel, dim3(tiles, (unsigned)splits), dim3(256), lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, s,
                     part, splits, B, r, scale, y, M, N);
  return hipGetLastError();
}

}  // namespace qlora
