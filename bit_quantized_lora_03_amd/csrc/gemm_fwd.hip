// Fused forward GEMM: y = x . deq(W)^T + (alpha/r) . (x . A^T) . B^T (gfx950).
//
// [QLoRA / infivelines.com]: the 4-bit base is dequantised to bf16 one block
// at a time inside the matrix multiply, and the adapters stay in full
// precision.  Here one 64-wide k tile of a weight row is exactly one NF4
// block, so each thread decodes one block per k tile into LDS with that
// block's own 16-entry table, and the tile feeds bf16 MFMA (32x32x16,
// fp32 accumulate) with the activation tile.
//
// The adapter term rides on the same accumulators: with xs = [hi | lo] the
// bf16 split of s . x . A^T (hi + lo equals the fp32 value to 2^-17), the
// product xs . [B | B]^T is run as 2r extra reduction columns after the
// base reduction, so y is rounded to bf16 exactly once.
//
// Block tile 256 (n) x 256 (m) x 64 (k); 4 waves in a 2 x 2 grid, each a
// 128 x 128 sub-tile as 4 x 4 MFMA tiles (256 accumulators per lane, one
// wave per SIMD).  LDS holds two stages of (W tile, x tile), 128 KiB; the
// next tile's global loads are in flight while the current one is
// multiplied.

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int TILE = 256;   // n and m extent of a block tile
constexpr int KT = 64;      // k extent of one stage (= one NF4 block)
constexpr int ROW_CHUNKS = KT / 8;              // 16-byte chunks per tile row
constexpr int TILE_CHUNKS = TILE * ROW_CHUNKS;  // u32x4 per tile

struct FwdParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* x;
  const uint16_t* xs;
  const uint16_t* B;
  uint16_t* y;
  int64_t M, N, K;
  int r;
  Nf4Levels L;
};

// Tile rows are 128 B; the 16-byte chunk index is xor-swizzled with the row
// so that 8 consecutive rows read at the same logical chunk hit 8 distinct
// chunk positions (all banks).
__device__ __forceinline__ int rk(int row, int chunk) { return row * ROW_CHUNKS + (chunk ^ (row & 7)); }

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(FwdParams p) {
  __shared__ u32x4_t lds[2][2][TILE_CHUNKS];  // [stage][0 = W, 1 = x]
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t n0 = (int64_t)blockIdx.x * TILE;
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

  // --- per-thread staging registers for one k tile ---
  u32x4_t xr[8];
  u32x4_t cr[2];
  float wscale;
  const int64_t wrow = n0 + t;          // this thread decodes W row n0 + t
  const bool wrow_ok = wrow < N;

  auto load_tile = [&](int64_t kt) {
    const int64_t k0 = kt * KT;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = m0 + (t >> 3) + 32 * j;
      xr[j] = (m < M) ? *reinterpret_cast<const u32x4_t*>(p.x + m * K + k0 + 8 * (t & 7)) : zero;
    }
    if (wrow_ok) {
      const int64_t idx = wrow * K + k0;  // first element of the block
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
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 8; ++j) lds[stage][1][rk((t >> 3) + 32 * j, t & 7)] = xr[j];
    const Nf4Lut lut = nf4_make_lut(p.L, wscale);
#pragma unroll
    for (int c = 0; c < 8; ++c) lds[stage][0][rk(t, c)] = nf4_decode8(lut, cr[c >> 2][c & 3]);
  };
  auto compute = [&](int stage) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = 2 * kk + lg;
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lds[stage][0][rk(128 * wn + 32 * i + lr, ch)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds[stage][1][rk(128 * wm + 32 * j + lr, ch)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  const int64_t nkt = K / KT;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nkt) load_tile(kt + 1);
    compute(cur);
    if (kt + 1 < nkt) store_tile(cur ^ 1);
    __syncthreads();
  }

  // --- adapter columns: xs [M, 2r] against [B | B] ---
  const int r = p.r;
  const int ext_tiles = (2 * r + KT - 1) / KT;
  for (int e = 0; e < ext_tiles; ++e) {
    const int64_t m = m0 + t;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = e * KT + 8 * c;
      u32x4_t wv = zero, xv = zero;
      if (col < 2 * r) {
        const int j = col < r ? col : col - r;
        if (wrow_ok) wv = *reinterpret_cast<const u32x4_t*>(p.B + wrow * r + j);
        if (m < M) xv = *reinterpret_cast<const u32x4_t*>(p.xs + m * 2 * r + col);
      }
      lds[0][0][rk(t, c)] = wv;
      lds[0][1][rk(t, c)] = xv;
    }
    __syncthreads();
    compute(0);
    __syncthreads();
  }

  // --- epilogue: D[n][m]; lane holds m = lr, n = 8(v/4) + 4 lg + v%4 ---
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + 128 * wm + 32 * j + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + 128 * wn + 32 * i + 8 * q + 4 * lg;
        if (n < N) {
          u32x2_t o;
          o[0] = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          o[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2_t*>(p.y + m * N + n) = o;
        }
      }
    }
  }
}

hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const uint16_t* x, const uint16_t* xs, const uint16_t* B,
                           uint16_t* y, int64_t M, int64_t N, int64_t K, int r,
                           const Nf4Levels& L, hipStream_t s) {
  FwdParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.x = x;
  p.xs = xs;
  p.B = B;
  p.y = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  p.L = L;
  dim3 grid((unsigned)((N + TILE - 1) / TILE), (unsigned)((M + TILE - 1) / TILE));
  hipLaunchKernelGGL(fwd_gemm_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
