// Fused forward GEMM: y = x . deq(W)^T + (alpha/r) . (x . A^T) . B^T (gfx950).
//
// [QLoRA / infivelines.com]: the 4-bit base is dequantised to bf16 one block
// at a time inside the matrix multiply, and the adapters stay in full
// precision.  One 64-wide k tile of a weight row is exactly one NF4 block,
// so each thread decodes one block per k tile into LDS with that block's own
// 16-entry table, and the tile feeds bf16 MFMA (32x32x16, fp32 accumulate)
// together with the activation tile.
//
// The adapter term rides on the same accumulators: with xs = [hi | lo] the
// bf16 split of s . x . A^T (hi + lo equals the fp32 value to 2^-17), the
// product xs . [B | B]^T runs as 2r extra reduction columns after the base
// reduction, so y is rounded to bf16 exactly once.
//
// Block tile 256 (n) x 256 (m) x 64 (k); 4 waves in a 2 x 2 grid, each a
// 128 x 128 sub-tile of 4 x 4 MFMA tiles (256 fp32 accumulators per lane,
// one wave per SIMD).  Two LDS stages of (W tile, x tile), 128 KiB.
//
// Pipeline per k tile: the MFMAs of tile t run from LDS stage t&1 while the
// same waves decode tile t+1's codes (loaded one tile earlier) into the
// other stage, one quarter of the decode after each quarter of the MFMAs,
// so the matrix cores and the vector ALUs work at the same time.  Codes are
// fetched two tiles ahead and x one tile ahead.  Out-of-range rows are
// clamped to the last valid row instead of branched around, so the loop
// body is a single basic block; their results are never stored.
//
// When the output has too few tiles to fill the chip, the k range is split
// over gridDim.z blocks that write fp32 partials; fwd_reduce adds them in a
// fixed order and rounds once.

#include <type_traits>

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
  uint16_t* y;     // bf16 output (splits == 1)
  float* part;     // fp32 partials [splits][M][N] (splits > 1)
  int64_t M, N, K;
  int r;
  int splits;
  Nf4Levels L;
};

// Tile rows are 128 B, so an even row covers banks 0..31 and an odd row
// banks 32..63.  A 16-byte read serves 16 lanes per LDS cycle, here 16
// consecutive rows at one logical chunk: xor-swizzling the chunk with
// (row / 2) mod 8 puts each pair of rows at its own chunk, so the 16 lanes
// cover all 64 banks once (swizzling with row mod 8 would map rows r and
// r + 8 to the same banks).
__device__ __forceinline__ int rk(int row, int chunk) {
  return row * ROW_CHUNKS + (chunk ^ ((row >> 1) & 7));
}

__device__ __forceinline__ int64_t clamp_row(int64_t v, int64_t hi) { return v < hi ? v : hi - 1; }

}  // namespace

// MS: 32-wide token subtiles per wave.  MS = 4 is the 256 (n) x 256 (m)
// block tile; MS = 2 halves the token extent (256 x 128), which doubles the
// number of output tiles for small-M shapes and so halves the k splits (and
// their fp32 partials) needed to fill the chip.
template <int MS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(FwdParams p) {
  constexpr int TM = 64 * MS;             // token rows of the block tile
  constexpr int XR = TM / 32;             // x rows staged per thread
  constexpr int WCH = TILE * ROW_CHUNKS;  // W stage, u32x4
  constexpr int XCH = TM * ROW_CHUNKS;    // x stage, u32x4
  __shared__ u32x4_t lds[2][WCH + XCH];   // [stage][W tile | x tile]
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m_tiles = (M + TM - 1) / TM, n_tiles = (N + TILE - 1) / TILE;
  const TileCoord tc = xcd_tile(blockIdx.x, (int64_t)gridDim.x, m_tiles, n_tiles, 4);
  const int64_t n0 = tc.n * TILE;
  const int64_t m0 = tc.m * TM;
  const int z = (int)tc.z;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto W = [&](int stage, int row, int chunk) -> u32x4_t& { return lds[stage][rk(row, chunk)]; };
  auto Xl = [&](int stage, int row, int chunk) -> u32x4_t& {
    return lds[stage][WCH + rk(row, chunk)];
  };

  // k tiles of this split
  const int64_t nkt = K / KT;
  const int64_t kt0 = nkt * z / p.splits, kt1 = nkt * (z + 1) / p.splits;

  f32x16_t acc[4][MS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MS; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // this thread decodes weight row n0 + t (clamped) and stages x rows
  // m0 + (t >> 3) + 32 j, chunk t & 7
  const int64_t wrow = clamp_row(n0 + t, N);
  const uint8_t* wcodes = p.codes + ((wrow * K) >> 1);
  const int64_t wblk0 = (wrow * K) >> 6;
  // x rows m0 + (t >> 3) + 32 j through a buffer descriptor: rows past M
  // read as zero
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(p.x, (uint32_t)(M * K * 2));
  const uint32_t xoff = (uint32_t)(((m0 + (t >> 3)) * K + 8 * (t & 7)) * 2);
  const uint32_t xrow_step = (uint32_t)(32 * K * 2);

  // The scale byte and its step stay raw until the tile is decoded (an
  // iteration later): forming s' here would make the wave wait for this
  // prefetch -- and, since loads return in order, for every load before it.
  struct Codes {
    u32x4_t c0, c1;
    uint32_t q;
    float st;
  };
  auto load_codes = [&](int64_t kt, Codes& c) {
    const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(wcodes + kt * (KT / 2));
    c.c0 = cp[0];
    c.c1 = cp[1];
    const int64_t b = wblk0 + kt;
    c.q = p.qscale[b];
    c.st = p.step[b >> 8];
  };
  auto load_x = [&](int64_t kt, u32x4_t (&xr)[XR]) {
    const uint32_t o = xoff + (uint32_t)(kt * KT * 2);
#pragma unroll
    for (int j = 0; j < XR; ++j) xr[j] = buffer_load16(xres, o + j * xrow_step);
  };
  auto store_x = [&](int stage, const u32x4_t (&xr)[XR]) {
#pragma unroll
    for (int j = 0; j < XR; ++j) Xl(stage, (t >> 3) + 32 * j, t & 7) = xr[j];
  };
  auto mfma_step = [&](int stage, int kk) {
    const int ch = 2 * kk + lg;
    u32x4_t a[4], b[MS];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = W(stage, 128 * wn + 32 * i + lr, ch);
#pragma unroll
    for (int j = 0; j < MS; ++j) b[j] = Xl(stage, 32 * MS * wm + 32 * j + lr, ch);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MS; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  };

  if (kt0 < kt1) {
    // Register sets are indexed by tile parity (relative to kt0): X[q] and
    // C[q] hold the x rows and codes of a tile with parity q.  At the top of
    // iteration kt the set of parity(kt) is free (tile kt already sits in
    // LDS), so tile kt+2 is loaded into it there; tile kt+1's set, loaded an
    // iteration earlier, is decoded and written into the other LDS stage.
    // The loop is unrolled by two so the parity is a constant and no
    // register holding an in-flight load is ever copied (a copy would make
    // the compiler wait for the load).  Prefetch indices are clamped into
    // the split, so loads are unconditional.
    const int64_t last = kt1 - 1;
    auto cl = [&](int64_t v) { return v < last ? v : last; };
    Codes C[2];
    u32x4_t X[2][XR];
    load_codes(kt0, C[0]);
    load_x(kt0, X[0]);
    store_x(0, X[0]);
    {
      const Nf4Lut lut = nf4_make_lut(p.L, nf4_block_scale(C[0].q, C[0].st));
#pragma unroll
      for (int c = 0; c < 8; ++c) W(0, t, c) = nf4_decode8(lut, (c < 4 ? C[0].c0 : C[0].c1)[c & 3]);
    }
    load_x(cl(kt0 + 1), X[1]);
    load_codes(cl(kt0 + 1), C[1]);
    __syncthreads();

    // Hand-scheduled iteration.  Issue is in order, so back-to-back MFMAs
    // would hold everything behind them; instead each MFMA of the tile is
    // followed by a small, fixed amount of other work and a scheduling
    // fence, so the vector work executes while the matrix core is busy.
    auto iteration = [&](int64_t kt, auto parity) {
      constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
      constexpr int SPK = 4 * MS;       // MFMAs (slots) per k step
      constexpr int NRD = 4 + MS;       // operand reads per k step
      // tile kt+2 into the free set (loads issued first, used an iteration later)
      load_x(cl(kt + 2), X[cur]);
      load_codes(cl(kt + 2), C[cur]);
      const Codes& cn = C[nxt];
      u32x4_t op[2][2][4];  // [buffer][a|b][i]
      auto read_op = [&](int kk, int buf, int q) {
        const int ch = 2 * kk + lg;
        if (q < 4)
          op[buf][0][q] = W(cur, 128 * wn + 32 * q + lr, ch);
        else
          op[buf][1][q - 4] = Xl(cur, 32 * MS * wm + 32 * (q - 4) + lr, ch);
      };
#pragma unroll
      for (int q = 0; q < NRD; ++q) read_op(0, 0, q);

      // Work units of the tile, in order: the table of tile kt+1's block
      // (units 0..7), the decode of its 8 code words (6 units each, about 5
      // vector ops per unit, the last one the 16-byte LDS write), the LDS
      // writes of its x rows (units 56..56+XR-1).  MS = 4 runs one unit per
      // MFMA (each fits in the MFMA's 32-cycle shadow), MS = 2 two.  The
      // operand reads of step kk+1 ride in the last slots of step kk.
      uint32_t pk[8];
      Nf4Lut lut;
      float sc = 0.0f;
      uint32_t dn0 = 0, dn1 = 0, nh = 0, pick = 0, la = 0, lb = 0;
      u32x4_t dv = zero;
      auto lookup_a = [&](uint32_t n) {  // low-byte planes of 4 codes
        nh = n & 0x07070707u;
        pick = ((n >> 1) & 0x04040404u) | 0x03020100u;
        la = perm(lut.lo[1], lut.lo[0], n);
        lb = perm(lut.lo[3], lut.lo[2], nh);
      };
      auto lookup_b = [&](uint32_t n, uint32_t& o01, uint32_t& o23) {  // high bytes, merge
        const uint32_t lo = perm(lb, la, pick);
        const uint32_t hi =
            perm(perm(lut.hi[3], lut.hi[2], nh), perm(lut.hi[1], lut.hi[0], n), pick);
        o01 = perm(hi, lo, 0x05010400u);
        o23 = perm(hi, lo, 0x07030602u);
      };
      auto unit = [&](int u) {
        if (u < 4) {
          if (u == 0) sc = nf4_block_scale(cn.q, cn.st);
          pk[2 * u] = pack_bf16x2(p.L.v[4 * u] * sc, p.L.v[4 * u + 1] * sc);
          pk[2 * u + 1] = pack_bf16x2(p.L.v[4 * u + 2] * sc, p.L.v[4 * u + 3] * sc);
        } else if (u < 8) {
          const int j = u - 4;
          lut.lo[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
          lut.hi[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
        } else if (u < 56) {
          const int c = (u - 8) / 6, w = (u - 8) % 6;
          const uint32_t v = (c < 4 ? cn.c0 : cn.c1)[c & 3];
          switch (w) {
            case 0: {
              const uint32_t ev = v & 0x0F0F0F0Fu, od = (v >> 4) & 0x0F0F0F0Fu;
              dn0 = perm(od, ev, 0x05010400u);  // codes 0..3 of the word, one per byte
              dn1 = perm(od, ev, 0x07030602u);  // codes 4..7
              break;
            }
            case 1: lookup_a(dn0); break;
            case 2: { uint32_t o0, o1; lookup_b(dn0, o0, o1); dv[0] = o0; dv[1] = o1; break; }
            case 3: lookup_a(dn1); break;
            case 4: { uint32_t o2, o3; lookup_b(dn1, o2, o3); dv[2] = o2; dv[3] = o3; break; }
            default: W(nxt, t, c) = dv; break;
          }
        } else if (u < 56 + XR) {
          // tile kt+1's x rows into the other stage
          Xl(nxt, (t >> 3) + 32 * (u - 56), t & 7) = X[nxt][u - 56];
        }
      };
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int s = 0; s < SPK; ++s) {
          const int i = s / MS, j = s % MS;
          acc[i][j] = mfma32x32x16(op[kk & 1][0][i], op[kk & 1][1][j], acc[i][j]);
          const int slot = SPK * kk + s;
          if (kk < 3 && s >= SPK - NRD) read_op(kk + 1, (kk + 1) & 1, s - (SPK - NRD));
          constexpr int UPS = 16 / SPK;  // units per slot: 64 units over 4 SPK slots
#pragma unroll
          for (int e = 0; e < UPS; ++e) unit(UPS * slot + e);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
    };
    for (int64_t kt = kt0; kt < kt1; kt += 2) {
      iteration(kt, std::integral_constant<int, 0>());
      if (kt + 1 < kt1) iteration(kt + 1, std::integral_constant<int, 1>());
    }
  }

  // --- adapter columns: xs [M, 2r] against [B | B] (last split only) ---
  const int r = p.r;
  if (z == p.splits - 1) {
    const int ext_tiles = (2 * r + KT - 1) / KT;
    const int64_t m = clamp_row(m0 + (t % TM), M);
    for (int e = 0; e < ext_tiles; ++e) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = e * KT + 8 * c;
        u32x4_t wv = zero, xv = zero;
        if (col < 2 * r) {
          const int j = col < r ? col : col - r;
          wv = *reinterpret_cast<const u32x4_t*>(p.B + wrow * r + j);
          xv = *reinterpret_cast<const u32x4_t*>(p.xs + m * 2 * r + col);
        }
        W(0, t, c) = wv;
        if (t < TM) Xl(0, t, c) = xv;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) mfma_step(0, kk);
      __syncthreads();
    }
  }

  // --- epilogue: D[n][m] -> y[m][n] (or the split's fp32 partial) ---
  __syncthreads();  // the LDS stages are free from here on
  float* scratch = reinterpret_cast<float*>(&lds[0][0]) + wave * kEpiFloats;
  store_acc_tile<MS>(acc, scratch, n0 + 128 * wn, m0 + 32 * MS * wm, N, M, p.splits > 1,
                     p.splits > 1 ? p.part + (int64_t)z * M * N : nullptr, p.y, N, lane);
}

// out[i] = bf16(sum_z part[z][i]), i over M*N (4 per thread), fixed order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t count,
                                                            uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < count; i += stride) {
    f32x4_t s = *reinterpret_cast<const f32x4_t*>(part + i);
    for (int z = 1; z < splits; ++z) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + (int64_t)z * count + i);
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
    u32x2_t o;
    o[0] = pack_bf16x2(s[0], s[1]);
    o[1] = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<u32x2_t*>(out + i) = o;
  }
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                                hipStream_t s) {
  int64_t g = (count / 4 + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)g), dim3(256), 0, s, part, splits,
                     count, out);
  return hipGetLastError();
}

// Block tile and k splits for an output of M x N with a reduction of Kred.
// For each token tile (256 or 128 rows) the k range is split until ~256
// blocks fill the chip (at least 4 k tiles per split); the choice is the
// smaller estimate of  flops / rate(tile) + the fp32 partials written and
// read back.  The rates are the measured sustained throughputs of the two
// tiles (the 256-row tile amortises each decoded weight over twice the
// tokens, the 128-row one needs half the splits).
GemmConfig gemm_config(int64_t M, int64_t N, int64_t Kred) {
  const int64_t nkt = Kred / KT;
  const int64_t n_t = (N + TILE - 1) / TILE;
  GemmConfig best{256, 1};
  double best_t = 1e300;
  for (int tm : {256, 128}) {
    const int64_t tiles = ((M + tm - 1) / tm) * n_t;
    int64_t s = tiles >= 192 ? 1 : 256 / tiles;
    if (s > nkt / 4) s = nkt / 4;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    const double blocks = (double)tiles * s;
    const double fill = blocks >= 256 ? 1.0 : blocks / 256.0;
    const double rate = (tm == 256 ? 1.1e15 : 0.8e15) * fill;  // flop/s
    const double partial = s > 1 ? 2.0 * s * (double)M * N * 4 / 5.0e12 : 0.0;
    const double est = 2.0 * M * N * Kred / rate + partial;
    if (est < best_t) {
      best_t = est;
      best = GemmConfig{tm, (int)s};
    }
  }
  return best;
}

int gemm_splits(int64_t M, int64_t N, int64_t Kred) { return gemm_config(M, N, Kred).splits; }

hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const uint16_t* x, const uint16_t* xs, const uint16_t* B,
                           uint16_t* y, float* part, int splits, int64_t M, int64_t N, int64_t K,
                           int r, const Nf4Levels& L, hipStream_t s) {
  const GemmConfig cfg = gemm_config(M, N, K);
  if (cfg.splits != splits) return hipErrorInvalidValue;  // workspace laid out for another split
  FwdParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.x = x;
  p.xs = xs;
  p.B = B;
  p.y = y;
  p.part = part;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  p.splits = splits;
  p.L = L;
  const int64_t blocks = ((N + TILE - 1) / TILE) * ((M + cfg.tm - 1) / cfg.tm) * splits;
  if (cfg.tm == 256)
    hipLaunchKernelGGL(fwd_gemm_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_gemm_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, M * N, y, s);
}

}  // namespace qlora
