// Fused backward GEMM for the input gradient (gfx950):
//     dX = dy . deq(W) + (alpha/r) . (dy . B) . A
//
// [QLoRA -- the democratization event, the recipe] / [QLoRA /
// infivelines.com]: gradients flow back through the frozen quantised base
// without updating it; the base is dequantised on the fly.
//
// The reduction here runs over the output features n, while the packed
// weight is stored k-contiguous (row n holds blocks along k).  Each block
// tile therefore decodes a 64 (n) x 256 (k) slab row by row -- one NF4
// block per thread, the same decode as the forward pass -- and writes it
// into LDS k-major (n contiguous), so that MFMA operands are again 16-byte
// reads.  dy tiles go to LDS as in the forward pass.
//
// The adapter term uses the same accumulators: with gs = [hi | lo] the bf16
// split of s . dy . B, gs . [A ; A] is run as 2r extra reduction rows.
//
// Block tile 256 (k) x 256 (m), 64 reduction rows per stage; 4 waves in a
// 2 x 2 grid of 128 x 128; two LDS stages of (W^T tile, dy tile), 128 KiB.

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int TILE = 256;
constexpr int RT = 64;  // reduction rows per stage
constexpr int ROW_CHUNKS = RT / 8;
constexpr int TILE_ELEMS = TILE * RT;

struct DxParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* dy;
  const uint16_t* gs;
  const uint16_t* A;
  uint16_t* dx;
  int64_t M, N, K;
  int r;
  Nf4Levels L;
};

// dy tile: [256 m][64 n], rows 128 B, chunk swizzled by row.
__device__ __forceinline__ int rk(int row, int chunk) { return row * ROW_CHUNKS + (chunk ^ (row & 7)); }

// W^T tile: [256 k][64 n] bf16, element offset.  The 16-byte n-chunk is
// swizzled by k's low 3 bits (8 consecutive k rows read at one chunk land
// in 8 distinct chunks) and by k's 64-block index (the four threads that
// decode one weight row at k, k+64, k+128, k+192 write distinct chunks).
__device__ __forceinline__ int wt_off(int k, int n) {
  const int chunk = (n >> 3) ^ (k & 7) ^ (((k >> 6) & 3) << 1);
  return k * RT + chunk * 8 + (n & 7);
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dx_gemm_kernel(DxParams p) {
  __shared__ uint16_t wt[2][TILE_ELEMS];
  __shared__ u32x4_t dyt[2][TILE * ROW_CHUNKS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wk = wave & 1, wm = wave >> 1;
  const int64_t k0 = (int64_t)blockIdx.x * TILE;
  const int64_t m0 = (int64_t)blockIdx.y * TILE;
  const int64_t M = p.M, N = p.N, K = p.K;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // this thread decodes reduction row (t >> 2) of the slab, k quarter (t & 3)
  const int wr = t >> 2;
  const int kq = t & 3;
  const int64_t kcol = k0 + 64 * kq;
  const bool kcol_ok = kcol < K;

  u32x4_t yr[8];
  u32x4_t cr[2];
  float wscale;

  auto load_tile = [&](int64_t st) {
    const int64_t nb = st * RT;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = m0 + (t >> 3) + 32 * j;
      yr[j] = (m < M) ? *reinterpret_cast<const u32x4_t*>(p.dy + m * N + nb + 8 * (t & 7)) : zero;
    }
    const int64_t n = nb + wr;
    if (kcol_ok) {
      const int64_t idx = n * K + kcol;  // first element of the block
      const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(p.codes + (idx >> 1));
      cr[0] = cp[0];
      cr[1] = cp[1];
      wscale = nf4_block_scale(p.qscale[idx >> 6], p.step[idx >> 14]);
    } else {
      cr[0] = zero;
      cr[1] = zero;
      wscale = 0.0f;
    }
  };
  // scatter 64 consecutive-k bf16 values of reduction row `wr` into W^T
  auto scatter_row = [&](int stage, const u32x4_t* v8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pr = v8[c][e];
        const int kl = 64 * kq + 8 * c + 2 * e;
        wt[stage][wt_off(kl, wr)] = (uint16_t)pr;
        wt[stage][wt_off(kl + 1, wr)] = (uint16_t)(pr >> 16);
      }
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dyt[stage][rk((t >> 3) + 32 * j, t & 7)] = yr[j];
    const Nf4Lut lut = nf4_make_lut(p.L, wscale);
    u32x4_t v8[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v8[c] = nf4_decode8(lut, cr[c >> 2][c & 3]);
    scatter_row(stage, v8);
  };
  auto compute = [&](int stage) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + lg;
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(&wt[stage][wt_off(128 * wk + 32 * i + lr, 8 * ch)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = dyt[stage][rk(128 * wm + 32 * j + lr, ch)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  const int64_t nst = N / RT;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int cur = (int)(st & 1);
    if (st + 1 < nst) load_tile(st + 1);
    compute(cur);
    if (st + 1 < nst) store_tile(cur ^ 1);
    __syncthreads();
  }

  // --- adapter rows: gs [M, 2r] against [A ; A] ---
  const int r = p.r;
  const int ext_tiles = (2 * r + RT - 1) / RT;
  for (int e = 0; e < ext_tiles; ++e) {
    // W^T side: reduction row c = e*64 + wr is A's row (c mod r), zero past 2r
    const int c = e * RT + wr;
    u32x4_t v8[8];
    const bool row_ok = c < 2 * r && kcol_ok;
    const int arow = c < r ? c : c - r;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      v8[q] = row_ok ? *reinterpret_cast<const u32x4_t*>(p.A + (int64_t)arow * K + kcol + 8 * q) : zero;
    scatter_row(0, v8);
    // dy side: rows m, columns c of gs
    const int64_t m = m0 + t;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = e * RT + 8 * q;
      dyt[0][rk(t, q)] = (m < M && col < 2 * r)
                             ? *reinterpret_cast<const u32x4_t*>(p.gs + m * 2 * r + col)
                             : zero;
    }
    __syncthreads();
    compute(0);
    __syncthreads();
  }

  // --- epilogue: D[k][m]; lane holds m = lr, k = 8(v/4) + 4 lg + v%4 ---
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + 128 * wm + 32 * j + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + 128 * wk + 32 * i + 8 * q + 4 * lg;
        if (k < K) {
          u32x2_t o;
          o[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          o[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2_t*>(p.dx + m * K + k) = o;
        }
      }
    }
  }
}

hipError_t launch_dx_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const uint16_t* dy, const uint16_t* gs, const uint16_t* A,
                          uint16_t* dx, int64_t M, int64_t N, int64_t K, int r,
                          const Nf4Levels& L, hipStream_t s) {
  DxParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.dy = dy;
  p.gs = gs;
  p.A = A;
  p.dx = dx;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  p.L = L;
  dim3 grid((unsigned)((K + TILE - 1) / TILE), (unsigned)((M + TILE - 1) / TILE));
  hipLaunchKernelGGL(dx_gemm_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
