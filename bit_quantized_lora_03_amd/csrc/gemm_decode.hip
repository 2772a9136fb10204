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
//    k span, so it builds that block's 16-entry bf16 table once and decodes
//    its 64 codes into the A operands of 8 consecutive MFMAs.  The reduction
//    order over k is permuted consistently for A and B (MFMA j of a span
//    sums k = base + 64 g + 8 j + e over g = 0, 1 and e = 0..7);
//  * the table lives in LDS, entry c of lane l of wave w at byte
//    4096 w + 256 c + 4 l, so a lookup is one v_perm (which places the
//    code, tagged with the wave, next to the lane's byte offset) and one
//    2-byte LDS read, and the 64 lanes of a read always hit 64 distinct
//    banks.  That is about two thirds of the vector work of resolving codes
//    with byte permutes in registers;
//  * x is small and stays in L2: each lane reads its token's 16-byte
//    operand pieces directly, two spans ahead;
//  * a block is 8 waves on 32 rows; each wave takes a contiguous eighth of
//    the block's k range and keeps the codes of the next 2 spans in flight
//    while it decodes the current 2.
//
// The adapter's down projection x . A^T rides along: rows of A (bf16, used
// as they are) form extra 32-row tiles whose partial sums land in columns
// N .. N+r-1 of the partial output.  Those tiles come first in the grid and
// are split finer over k, so they finish early instead of trailing.
//
// Grid: 1-D over (A tiles x SA splits) then (weight tiles x SW splits),
// ordered so that consecutive ranks share an XCD (workgroups are dealt to
// the 8 XCDs round-robin): the blocks of neighbouring row tiles run behind
// one L2.  Partial sums go to part[S][M][N + r] (S = max(SW, SA));
// decode_reduce adds them in a fixed order, forms the fp32 adapter term
// (alpha/r) . (x . A^T) . B^T and rounds y to bf16 once.

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int WAVES = 8;    // waves per block
constexpr int SPAN = 128;   // k per span (two 64-weight blocks per row)
constexpr int BATCH = 2;    // spans whose codes are requested together
constexpr int kTabBytes = WAVES * 16 * 64 * 4;  // per-lane NF4 tables, 32 KiB

struct DecodeParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* x;
  const uint16_t* A;
  float* part;
  int64_t M, N, K;
  int r;
  int sw, sa;          // k splits of the weight tiles and of the A tiles
  int64_t a_blocks;    // A tiles x sa (they come first)
  int64_t blocks;      // a_blocks + weight tiles x sw
  Nf4Levels L;
};

// codes of one span plus the raw scale byte and step: s' is formed only when
// the span is decoded, so that issuing the loads never waits for them
struct Span {
  u32x4_t c[2];
  uint32_t q;
  float st;
  bool ok;  // false: past the range, decodes to zeros
};

}  // namespace

__global__ __launch_bounds__(WAVES * 64) void decode_main_kernel(DecodeParams p) {
  // the tables are the kernel's only LDS (at offset 0, so a lookup address
  // needs no base added); after the main loop the space holds the reduction
  __shared__ __align__(16) uint8_t lds[kTabBytes];

  const int64_t id = blockIdx.x, per_xcd = (int64_t)gridDim.x / 8;
  const int64_t rank = (id % 8) * per_xcd + id / 8;  // grid padded to a multiple of 8
  if (rank >= p.blocks) return;
  const bool a_tile = rank < p.a_blocks;
  const int splits = a_tile ? p.sa : p.sw;
  const int64_t lr_rank = a_tile ? rank : rank - p.a_blocks;
  const int64_t tile = lr_rank / splits;
  const int z = (int)(lr_rank % splits);

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t n0 = tile * 32;
  const int64_t nrows = a_tile ? p.r : N;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // this wave's spans: the block's share of k, cut in contiguous eighths
  const int64_t spans_total = (K + SPAN - 1) / SPAN;
  const int64_t bs0 = spans_total * z / splits, bs1 = spans_total * (z + 1) / splits;
  const int64_t per_w = (bs1 - bs0 + WAVES - 1) / WAVES;
  const int64_t s_begin = bs0 + wave * per_w < bs1 ? bs0 + wave * per_w : bs1;
  const int64_t s_end = s_begin + per_w < bs1 ? s_begin + per_w : bs1;
  const int64_t n = n0 + lr;
  const bool row_ok = n < nrows;
  const bool tok_ok = lr < M;
  const uint16_t* xrow = p.x + (tok_ok ? lr : 0) * K;

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  // x operands.  Only the M token lanes load (the other lanes' columns of
  // the product are never stored, whatever their registers hold); spans past
  // the range read span 0, whose weights decode to zero.  The values are used
  // as loaded, so nothing waits for them before the MFMA that needs them.
  auto load_x = [&](int64_t sp, u32x4_t (&xb)[8]) {
    const int64_t kb = sp * SPAN + 64 * lg;
    const bool ok = sp < s_end && kb < K;
    const uint16_t* xp = xrow + (ok ? kb : 0);
    if (tok_ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[j] = *reinterpret_cast<const u32x4_t*>(xp + 8 * j);
    }
  };

  if (!a_tile) {
    // Loads are unconditional (a span out of range reads the row's first
    // block and is decoded with a zero scale), so no branch separates them
    // and they all stay in flight together.
    const uint8_t* row_codes = p.codes + (((row_ok ? n : 0) * K) >> 1);
    const int64_t row_blk = ((row_ok ? n : 0) * K) >> 6;
    auto load_span = [&](int64_t sp, Span& S) {
      const int64_t kb = sp * SPAN + 64 * lg;
      const bool ok = row_ok && sp < s_end && kb < K;
      const int64_t kk = ok ? kb : 0;
      const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(row_codes + (kk >> 1));
      S.c[0] = cp[0];
      S.c[1] = cp[1];
      const int64_t b = row_blk + (kk >> 6);
      S.q = p.qscale[b];
      S.st = p.step[b >> 8];
      S.ok = ok;
    };
    uint16_t* tab_w = reinterpret_cast<uint16_t*>(lds) + wave * 2048 + lane * 2;
    const uint32_t wtag = (uint32_t)wave * 0x10101010u;  // wave in bits 4..6 of each code byte
    const uint32_t lane4 = (uint32_t)lane * 4u;
    auto decode_span = [&](const Span& S, const u32x4_t (&xb)[8]) {
      // this lane's block table: entry c = bf16_rne(fp32(L[c] * s'))
      const float sc = S.ok ? nf4_block_scale(S.q, S.st) : 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t pk = pack_bf16x2(p.L.v[2 * q] * sc, p.L.v[2 * q + 1] * sc);
        tab_w[(2 * q) * 128] = (uint16_t)pk;
        tab_w[(2 * q + 1) * 128] = (uint16_t)(pk >> 16);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t v = S.c[j >> 2][j & 3];
        const uint32_t ev = (v & 0x0F0F0F0Fu) | wtag;
        const uint32_t od = ((v >> 4) & 0x0F0F0F0Fu) | wtag;
        const uint32_t q4[2] = {perm(od, ev, 0x05010400u), perm(od, ev, 0x07030602u)};
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // byte 0: the lane's offset, byte 1: code + 16 wave -> LDS address
          const uint32_t addr = perm(q4[e >> 2], lane4, 0x0C0C0000u | ((4u + (e & 3)) << 8));
          h[e] = *reinterpret_cast<const uint16_t*>(lds + addr);
        }
        u32x4_t a;
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = h[2 * q] | (h[2 * q + 1] << 16);
        acc = mfma32x32x16(a, xb[j], acc);
      }
    };

    // codes: batches of 2 spans in two register sets (batch b + 1 in flight
    // while batch b decodes); x: two spans ahead in four register sets
    // (span u of a batch of parity q uses set 2 q + u)
    Span C0[BATCH], C1[BATCH];
    u32x4_t X[2 * BATCH][8];
#pragma unroll
    for (int u = 0; u < 2 * BATCH; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) X[u][j] = zero;
    const int64_t nb = (s_end - s_begin + BATCH - 1) / BATCH;
    auto load_batch = [&](int64_t b, Span (&C)[BATCH]) {
#pragma unroll
      for (int u = 0; u < BATCH; ++u) load_span(s_begin + b * BATCH + u, C[u]);
    };
    auto run_batch = [&](int64_t b, const Span (&C)[BATCH], auto parity) {
      constexpr int q = decltype(parity)::value;
      const int64_t sp = s_begin + b * BATCH;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        load_x(sp + u + 2, X[(2 * q + u + 2) % 4]);
        if (sp + u < s_end) decode_span(C[u], X[2 * q + u]);
      }
    };
    if (nb > 0) {
      load_batch(0, C0);
      load_x(s_begin, X[0]);
      load_x(s_begin + 1, X[1]);
    }
    for (int64_t b = 0; b < nb; b += 2) {
      if (b + 1 < nb) load_batch(b + 1, C1);
      run_batch(b, C0, std::integral_constant<int, 0>());
      if (b + 1 < nb) {
        if (b + 2 < nb) load_batch(b + 2, C0);
        run_batch(b + 1, C1, std::integral_constant<int, 1>());
      }
    }
  } else {
    // rows of A: bf16 operands as stored
    const uint16_t* arow = p.A + (row_ok ? n : 0) * K;
    for (int64_t sp = s_begin; sp < s_end; ++sp) {
      const int64_t kb = sp * SPAN + 64 * lg;
      const bool ok = row_ok && kb < K;
      u32x4_t xb[8], av[8];
      load_x(sp, xb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        av[j] = ok ? *reinterpret_cast<const u32x4_t*>(arow + kb + 8 * j) : zero;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = mfma32x32x16(av[j], xb[j], acc);
    }
  }

  // ---- sum the 8 waves' tiles in LDS (wave order), write the partial ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [8][32 rows][M], M <= 32
  const int mcols = (int)M;
  // D[n][m]: lane holds token m = lr, rows n = 8(v/4) + 4 lg + v%4
  if (tok_ok) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      red[(wave * 32 + 8 * (v >> 2) + 4 * lg + (v & 3)) * mcols + lr] = acc[v];
  }
  __syncthreads();
  const int64_t col0 = a_tile ? N + n0 : n0;
  const int64_t ldp = N + p.r;
  for (int e = t; e < 32 * mcols; e += WAVES * 64) {
    const int m = e >> 5, row = e & 31;  // consecutive threads: consecutive columns
    if (n0 + row < nrows) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += red[(w * 32 + row) * mcols + m];
      p.part[((int64_t)z * M + m) * ldp + col0 + row] = s;
    }
  }
}

// sum over splits z = 0 .. splits-1 in order, eight loads issued at a time
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int64_t stride,
                                            int splits) {
  float s = 0.0f;
  for (int z0 = 0; z0 < splits; z0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = z0 + u < splits ? part[(int64_t)(z0 + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) s += v[u];
  }
  return s;
}

// y[m][n] = bf16( sum_z part[z][m][n] + scale * sum_j xa[m][j] B[n][j] ) with
// xa[m][j] = sum_z part[z][m][N + j]; fixed summation orders.  Block of 256
// threads = 64 columns n x 4 token groups.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part,
                                                            int sw, int sa,
                                                            const uint16_t* __restrict__ B,
                                                            int r, float scale,
                                                            uint16_t* __restrict__ y, int64_t M,
                                                            int64_t N) {
  __shared__ float xa[32 * 256];
  const int t = threadIdx.x;
  const int64_t ldp = N + r;
  for (int e = t; e < M * r; e += 256) {
    const int64_t m = e / r, j = e - m * r;
    xa[e] = sum_splits(part + m * ldp + N + j, M * ldp, sa);
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
      float acc = sum_splits(part + m * ldp + n, M * ldp, sw);
      acc += scale * lsum[i];
      y[m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
  }
}

namespace {

// k splits of the weight tiles: the fewest that keep the chip's 256 CUs
// (one 8-wave block each) evenly busy -- rounds of blocks times work per
// block, plus a small cost per split -- with at least one span per wave.
int weight_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + 31) / 32;
  const int64_t spans = (K + SPAN - 1) / SPAN;
  int best = 1;
  double best_cost = 1e30;
  for (int s = 1; s <= 8; ++s) {
    if (s > 1 && spans / s < WAVES) break;
    const int64_t rounds = (tiles * s + 255) / 256;
    const double cost = (double)rounds / s * (1.0 + 0.03 * s);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

// the A tiles are few and carry 4x the bytes per row: split them finer
int a_splits(int64_t K) {
  const int64_t spans = (K + SPAN - 1) / SPAN;
  int s = 8;
  while (s > 1 && spans / s < WAVES) --s;
  return s;
}

}  // namespace

int decode_splits(int64_t M, int64_t N, int64_t K) {
  (void)M;
  const int sw = weight_splits(N, K), sa = a_splits(K);
  return sw > sa ? sw : sa;
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
  p.sw = weight_splits(N, K);
  p.sa = a_splits(K);
  if (p.sw > splits || p.sa > splits) return hipErrorInvalidValue;  // workspace sized for fewer
  p.a_blocks = (int64_t)((r + 31) / 32) * p.sa;
  p.blocks = p.a_blocks + ((N + 31) / 32) * p.sw;
  p.L = L;
  const int64_t grid = (p.blocks + 7) / 8 * 8;
  hipLaunchKernelGGL(decode_main_kernel, dim3((unsigned)grid), dim3(WAVES * 64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, s,
                     part, p.sw, p.sa, B, r, scale, y, M, N);
  return hipGetLastError();
}

}  // namespace qlora
