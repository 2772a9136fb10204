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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(FwdParams p) {
  __shared__ u32x4_t lds[2][2][TILE_CHUNKS];  // [stage][0 = W, 1 = x]
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m_tiles = (M + TILE - 1) / TILE, n_tiles = (N + TILE - 1) / TILE;
  const TileCoord tc = xcd_tile(blockIdx.x, (int64_t)gridDim.x, m_tiles, n_tiles, 4);
  const int64_t n0 = tc.n * TILE;
  const int64_t m0 = tc.m * TILE;
  const int z = (int)tc.z;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // k tiles of this split
  const int64_t nkt = K / KT;
  const int64_t kt0 = nkt * z / p.splits, kt1 = nkt * (z + 1) / p.splits;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
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
  auto load_x = [&](int64_t kt, u32x4_t (&xr)[8]) {
    const uint32_t o = xoff + (uint32_t)(kt * KT * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) xr[j] = buffer_load16(xres, o + j * xrow_step);
  };
  auto store_x = [&](int stage, const u32x4_t (&xr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) lds[stage][1][rk((t >> 3) + 32 * j, t & 7)] = xr[j];
  };
  auto mfma_step = [&](int stage, int kk) {
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
    u32x4_t X[2][8];
    load_codes(kt0, C[0]);
    load_x(kt0, X[0]);
    store_x(0, X[0]);
    {
      const Nf4Lut lut = nf4_make_lut(p.L, nf4_block_scale(C[0].q, C[0].st));
#pragma unroll
      for (int c = 0; c < 8; ++c)
        lds[0][0][rk(t, c)] = nf4_decode8(lut, (c < 4 ? C[0].c0 : C[0].c1)[c & 3]);
    }
    load_x(cl(kt0 + 1), X[1]);
    load_codes(cl(kt0 + 1), C[1]);
    __syncthreads();

    // Hand-scheduled iteration.  Issue is in order, so back-to-back MFMAs
    // would hold everything behind them; instead each of the 64 MFMAs of a
    // tile is followed by one small unit of other work and a scheduling
    // fence: the next k-step's operand reads, a slice of the decode of tile
    // kt+1 into the other stage, its LDS writes.  The vector work then
    // executes while the matrix core is busy.
    auto iteration = [&](int64_t kt, auto parity) {
      constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
      // tile kt+2 into the free set (loads issued first, used an iteration later)
      load_x(cl(kt + 2), X[cur]);
      load_codes(cl(kt + 2), C[cur]);
      const Codes& cn = C[nxt];
      u32x4_t op[2][2][4];  // [buffer][a|b][i]
      auto read_ops = [&](int kk, int buf, int which, int i) {
        const int ch = 2 * kk + lg;
        if (which == 0)
          op[buf][0][i] = lds[cur][0][rk(128 * wn + 32 * i + lr, ch)];
        else
          op[buf][1][i] = lds[cur][1][rk(128 * wm + 32 * i + lr, ch)];
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        read_ops(0, 0, 0, i);
        read_ops(0, 0, 1, i);
      }
      // The 64 MFMA slots of the tile carry, in order: the table of tile
      // kt+1's block (slots 0..7), the decode of its 8 code words (6 slots
      // each, about 5 vector ops per slot, then the 16-byte LDS write), and
      // the LDS writes of its x rows (slots 56..63).  Each slot's vector work
      // fits in the shadow of one MFMA (32 cycles); the operand reads of
      // step kk+1 ride in slots 8..15 of step kk.
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
      auto unit = [&](int kk, int s) {
        const int slot = 16 * kk + s;
        // operand reads for step kk+1 in slots 8..15
        if (kk < 3 && s >= 8) read_ops(kk + 1, (kk + 1) & 1, (s - 8) >> 2, (s - 8) & 3);
        if (slot < 4) {
          if (slot == 0) sc = nf4_block_scale(cn.q, cn.st);
          pk[2 * slot] = pack_bf16x2(p.L.v[4 * slot] * sc, p.L.v[4 * slot + 1] * sc);
          pk[2 * slot + 1] = pack_bf16x2(p.L.v[4 * slot + 2] * sc, p.L.v[4 * slot + 3] * sc);
        } else if (slot < 8) {
          const int j = slot - 4;
          lut.lo[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
          lut.hi[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
        } else if (slot < 56) {
          const int c = (slot - 8) / 6, u = (slot - 8) % 6;
          const uint32_t v = (c < 4 ? cn.c0 : cn.c1)[c & 3];
          switch (u) {
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
            default: lds[nxt][0][rk(t, c)] = dv; break;
          }
        } else {
          // tile kt+1's x rows into the other stage
          lds[nxt][1][rk((t >> 3) + 32 * (slot - 56), t & 7)] = X[nxt][slot - 56];
        }
      };
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int i = s >> 2, j = s & 3;
          acc[i][j] = mfma32x32x16(op[kk & 1][0][i], op[kk & 1][1][j], acc[i][j]);
          unit(kk, s);
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
    const int64_t m = clamp_row(m0 + t, M);
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
        lds[0][0][rk(t, c)] = wv;
        lds[0][1][rk(t, c)] = xv;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) mfma_step(0, kk);
      __syncthreads();
    }
  }

  // --- epilogue: D[n][m] -> y[m][n] (or the split's fp32 partial) ---
  __syncthreads();  // the LDS stages are free from here on
  float* scratch = reinterpret_cast<float*>(&lds[0][0][0]) + wave * kEpiFloats;
  store_acc_tile(acc, scratch, n0 + 128 * wn, m0 + 128 * wm, N, M, p.splits > 1,
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

// Split the k range when the output tiles alone cannot fill the chip:
// aim for ~256 blocks, at least 4 k tiles per split.
int gemm_splits(int64_t M, int64_t N, int64_t Kred) {
  const int64_t tiles = ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
  const int64_t nkt = Kred / KT;
  if (tiles >= 192) return 1;
  int64_t s = 256 / tiles;
  if (s > nkt / 4) s = nkt / 4;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const uint16_t* x, const uint16_t* xs, const uint16_t* B,
                           uint16_t* y, float* part, int splits, int64_t M, int64_t N, int64_t K,
                           int r, const Nf4Levels& L, hipStream_t s) {
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
  const int64_t blocks = ((N + TILE - 1) / TILE) * ((M + TILE - 1) / TILE) * splits;
  hipLaunchKernelGGL(fwd_gemm_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, M * N, y, s);
}

}  // namespace qlora
