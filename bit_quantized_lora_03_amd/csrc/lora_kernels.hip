// Rank-r kernels of the LoRA path (gfx950, bf16 MFMA, fp32 accumulate).
//
// The adapter term y += s . (x . A^T) . B^T and its gradients are skinny
// products with one side equal to the rank r ("QLoRA -- Module 12.4",
// "Hugging Face + BitsAndBytes": LoraConfig(r, lora_alpha); s = alpha / r).
//
//  * lora_proj: out = split(s . X . Y^T), X [M, Kred] bf16 and Y either
//    [r, Kred] (A, for x . A^T) or [Kred, r] (B, for dy . B).  split(v)
//    stores hi = bf16(v) and lo = bf16(v - hi) as out[m][j] and
//    out[m][r + j]; hi + lo equals the fp32 value to 2^-17 relative, so the
//    rank-r product can ride on bf16 MFMA inside the fused GEMMs.  A second
//    copy, outT [2r][Mp] (tokens contiguous, Mp = M rounded up to 32, zero
//    past M), feeds lora_grad.
//  * lora_grad: C (+)= G^T . (S_hi + S_lo) with the reduction over the
//    tokens: dB [N, r] = dy^T . xs and dA [r, K] = gs^T . x.
//
// Both are latency-bound at the shapes of the layer (a few MB per call), so
// the reduction is spread over many small blocks: the waves of a block take
// interleaved shares of its range and are added in LDS in wave order; when
// a range is split over blocks, each block writes an fp32 partial and a
// finalize kernel adds the partials in split order.  Results are therefore
// deterministic.  Each wave keeps its next share's global loads in flight
// while it works on the current one, and two jobs share one launch.

#include "device_common.h"
#include "launch.h"

namespace qlora {

__device__ __forceinline__ uint16_t bf16_rne_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

__host__ __device__ __forceinline__ int64_t pad32(int64_t M) { return (M + 31) / 32 * 32; }

// Store the bf16 pair of v for (m, j) in both layouts (m < Mp; rows past M
// only get zeros in the transposed copy).
__device__ __forceinline__ void put_split(const LoraProjJob& J, int64_t M, int r, int64_t m,
                                          int j, float v) {
  const int64_t Mp = pad32(M);
  uint16_t hi = 0, lo = 0;
  if (m < M) {
    hi = bf16_rne_bits(v);
    lo = bf16_rne_bits(v - bf16_bits_to_f32(hi));  // v - hi is exact
    J.out[m * 2 * r + j] = hi;
    J.out[m * 2 * r + r + j] = lo;
  }
  J.outT[(int64_t)j * Mp + m] = hi;
  J.outT[(int64_t)(r + j) * Mp + m] = lo;
}

// ---------------------------------------------------------------------------
// lora_proj: grid (sum over jobs of ceil(M/64) * ceil(r/(16 JT)) * splits),
// 256 threads.  A block owns 64 tokens x 16 JT rank columns of one job and
// the z-th share of that job's reduction (jobs split in proportion to their
// reduction length, so their blocks carry equal work); wave w owns tokens
// 16 w .. 16 w + 15 and runs the block's whole k share with 16x16x32 MFMA.
// The token operand is one 16-byte load per lane (8 consecutive k of a
// row), straight from global memory, and so is A's operand per 16-column
// group (the four waves read the same A pieces, which stay in L1).  B
// ([Kred, r]) has k as its slow index, so the block loads it as 16-byte row
// pieces (8 rank columns of one k), turns them around once in a shared,
// double-buffered LDS tile per batch of k steps, and every wave reads its
// operands from there.  With one split the waves write the bf16 pairs
// themselves; otherwise they write fp32 partials P[z][m][j] and
// lora_proj_finalize adds the shares in order.
// ---------------------------------------------------------------------------
constexpr int kProjBatch = 4;  // k steps per register set
constexpr int kProjTRow = 40;  // transposed B row: 32 k + 8 pad (bf16), 80 bytes

template <int JT>
__global__ __launch_bounds__(256) void lora_proj_kernel(LoraProjJob j0, LoraProjJob j1,
                                                        int64_t blocks0, int64_t M, int r,
                                                        float scale) {
  __shared__ __align__(16) uint16_t tb[2][kProjBatch][16 * JT * kProjTRow];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraProjJob J = second ? j1 : j0;
  const int splits = J.splits;

  const int jblocks = (r + 16 * JT - 1) / (16 * JT);
  const int64_t b0 = second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
  const int z = (int)(b0 % splits);
  const int64_t bb = b0 / splits;
  const int64_t mblk = (bb / jblocks) * 64;
  const int64_t m0 = mblk + 16 * wave;
  const int jc = (int)(bb % jblocks) * 16 * JT;
  const int i = lane & 15, kg = lane >> 4;
  const int64_t m = m0 + i;
  const bool mok = m < M;
  const int64_t Kred = J.Kred;
  const int64_t nsteps = Kred / 32;
  const int64_t st0 = nsteps * z / splits, st1 = nsteps * (z + 1) / splits;
  const int64_t ns = st1 - st0;
  const int64_t nb = (ns + kProjBatch - 1) / kProjBatch;
  const uint16_t* xrow = J.X + (mok ? m : 0) * Kred + 8 * kg;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  f32x4_t acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto load_x = [&](int64_t bi, u32x4_t (&xv)[kProjBatch]) {
#pragma unroll
    for (int u = 0; u < kProjBatch; ++u) {
      const int64_t s = bi * kProjBatch + u;
      xv[u] = (mok && s < ns) ? *reinterpret_cast<const u32x4_t*>(xrow + 32 * (st0 + s)) : zero;
    }
  };

  if (!J.kmajor) {
    // A [r, Kred]: row pieces are MFMA operands as they are
    auto load_a = [&](int64_t bi, u32x4_t (&yv)[kProjBatch][JT]) {
#pragma unroll
      for (int u = 0; u < kProjBatch; ++u) {
        const int64_t s = bi * kProjBatch + u;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const int jj = jc + 16 * jt + i;
          yv[u][jt] = (jj < r && s < ns)
                          ? *reinterpret_cast<const u32x4_t*>(J.Y + (int64_t)jj * Kred +
                                                              32 * (st0 + s) + 8 * kg)
                          : zero;
        }
      }
    };
    auto mma = [&](const u32x4_t (&xv)[kProjBatch], const u32x4_t (&yv)[kProjBatch][JT]) {
#pragma unroll
      for (int u = 0; u < kProjBatch; ++u)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) acc[jt] = mfma16x16x32(xv[u], yv[u][jt], acc[jt]);
    };
    u32x4_t X0[kProjBatch], X1[kProjBatch], Y0[kProjBatch][JT], Y1[kProjBatch][JT];
    if (nb > 0) {
      load_x(0, X0);
      load_a(0, Y0);
    }
    for (int64_t bi = 0; bi < nb; bi += 2) {
      if (bi + 1 < nb) {
        load_x(bi + 1, X1);
        load_a(bi + 1, Y1);
      }
      mma(X0, Y0);
      if (bi + 1 < nb) {
        if (bi + 2 < nb) {
          load_x(bi + 2, X0);
          load_a(bi + 2, Y0);
        }
        mma(X1, Y1);
      }
    }
  } else {
    // B [Kred, r]: thread t loads JT row pieces per batch, piece p = t + 256 q:
    // step p / (64 JT), k row (p mod 64 JT) / (2 JT), columns 8 (p mod 2 JT)
    auto load_b = [&](int64_t bi, u32x4_t (&br)[JT]) {
#pragma unroll
      for (int q = 0; q < JT; ++q) {
        const int pc = t + 256 * q;
        const int u = pc / (64 * JT), w = pc % (64 * JT);
        const int kr = w / (2 * JT), cp = w % (2 * JT);
        const int64_t s = bi * kProjBatch + u;
        const int col = jc + 8 * cp;
        br[q] = (col < r && s < ns)
                    ? *reinterpret_cast<const u32x4_t*>(J.Y + (32 * (st0 + s) + kr) * r + col)
                    : zero;
      }
    };
    auto put_b = [&](int buf, const u32x4_t (&br)[JT]) {
#pragma unroll
      for (int q = 0; q < JT; ++q) {
        const int pc = t + 256 * q;
        const int u = pc / (64 * JT), w = pc % (64 * JT);
        const int kr = w / (2 * JT), cp = w % (2 * JT);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tb[buf][u][(8 * cp + e) * kProjTRow + kr] = (uint16_t)(br[q][e >> 1] >> (16 * (e & 1)));
      }
    };
    auto mma = [&](int buf, const u32x4_t (&xv)[kProjBatch]) {
#pragma unroll
      for (int u = 0; u < kProjBatch; ++u)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const u32x4_t b =
              *reinterpret_cast<const u32x4_t*>(&tb[buf][u][(16 * jt + i) * kProjTRow + 8 * kg]);
          acc[jt] = mfma16x16x32(xv[u], b, acc[jt]);
        }
    };
    // Batch b's pieces go into buffer b & 1 after the barrier of batch b - 1,
    // which every wave reaches only once it is done reading batch b - 2 (the
    // same buffer); all waves run the same number of batches.
    u32x4_t X0[kProjBatch], X1[kProjBatch], B0[JT], B1[JT];
    if (nb > 0) {
      load_x(0, X0);
      load_b(0, B0);
    }
    for (int64_t bi = 0; bi < nb; bi += 2) {
      if (bi + 1 < nb) {
        load_x(bi + 1, X1);
        load_b(bi + 1, B1);
      }
      put_b(0, B0);
      __syncthreads();
      mma(0, X0);
      if (bi + 1 < nb) {
        if (bi + 2 < nb) {
          load_x(bi + 2, X0);
          load_b(bi + 2, B0);
        }
        put_b(1, B1);
        __syncthreads();
        mma(1, X1);
      }
    }
  }

  // D[token][j]: lane holds column j = lane % 16, tokens 4 (lane / 16) + v
  const int64_t Mp = pad32(M);
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int jo = jc + 16 * jt + i;
    if (jo >= r) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mo = m0 + 4 * kg + v;
      if (splits == 1) {
        if (mo < Mp) put_split(J, M, r, mo, jo, scale * acc[jt][v]);
      } else if (mo < M) {
        J.P[((int64_t)z * M + mo) * r + jo] = acc[jt][v];
      }
    }
  }
}

// bf16 pairs of scale * sum_z P[z] (z in order); grid-stride over both
// jobs' Mp x r values (rows past M get zeros in the transposed copy).
__global__ __launch_bounds__(256) void lora_proj_finalize_kernel(LoraProjJob j0, LoraProjJob j1,
                                                                 int njobs, int64_t M, int r,
                                                                 float scale) {
  const int64_t per = pad32(M) * r, total = per * njobs;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const bool second = e >= per;
    const LoraProjJob J = second ? j1 : j0;
    const int splits = J.splits;
    if (splits == 1) continue;  // the job's blocks wrote their results themselves
    const int64_t ee = second ? e - per : e;
    const int64_t m = ee / r;
    const int j = (int)(ee - m * r);
    float sum = 0.0f;
    if (m < M) {
      float v[16];
#pragma unroll
      for (int z = 0; z < 16; ++z) v[z] = z < splits ? J.P[((int64_t)z * M + m) * r + j] : 0.0f;
      sum = v[0];
#pragma unroll
      for (int z = 1; z < 16; ++z)
        if (z < splits) sum += v[z];
    }
    put_split(J, M, r, m, j, scale * sum);
  }
}

static int proj_jt(int r) { return r <= 16 ? 1 : (r <= 32 ? 2 : 4); }

// k splits of one or two jobs sharing a launch: about 512 blocks in all,
// each job's splits in proportion to its reduction length (equal work per
// block), at least 8 k steps per split.
void lora_proj_plan(int64_t M, int r, int64_t K0, int64_t K1, int& s0, int& s1) {
  const int jw = 16 * proj_jt(r);
  const int64_t tiles = ((M + 63) / 64) * ((r + jw - 1) / jw);
  const double total_k = (double)K0 + (double)K1;
  auto pick = [&](int64_t Kred) {
    if (Kred <= 0 || tiles == 0) return 1;
    int64_t s = (int64_t)(512.0 * (double)Kred / (total_k * (double)tiles) + 0.5);
    if (s > Kred / 256) s = Kred / 256;
    if (s > kProjMaxSplits) s = kProjMaxSplits;
    return s < 1 ? 1 : (int)s;
  };
  s0 = pick(K0);
  s1 = pick(K1);
}

hipError_t launch_lora_proj(const LoraProjJob& j0, const LoraProjJob* j1, int64_t M, int r,
                            float scale, hipStream_t s) {
  const int njobs = j1 ? 2 : 1;
  const int jt = proj_jt(r);
  const int jw = 16 * jt;
  // ceil(M/64) token blocks cover every row of the transposed copy (Mp =
  // M rounded up to 32 <= the blocks' extent); rows past Mp are not written
  const int64_t tiles = ((M + 63) / 64) * ((r + jw - 1) / jw);
  const LoraProjJob jb = j1 ? *j1 : j0;
  const int64_t blocks0 = tiles * j0.splits, blocks1 = j1 ? tiles * j1->splits : 0;
  if (blocks0 + blocks1 == 0) return hipSuccess;
  const dim3 grid((unsigned)(blocks0 + blocks1));
  if (jt == 1)
    hipLaunchKernelGGL(lora_proj_kernel<1>, grid, dim3(256), 0, s, j0, jb, blocks0, M, r, scale);
  else if (jt == 2)
    hipLaunchKernelGGL(lora_proj_kernel<2>, grid, dim3(256), 0, s, j0, jb, blocks0, M, r, scale);
  else
    hipLaunchKernelGGL(lora_proj_kernel<4>, grid, dim3(256), 0, s, j0, jb, blocks0, M, r, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (j0.splits == 1 && (!j1 || j1->splits == 1))) return e;
  int64_t g = (pad32(M) * r * njobs + 255) / 256;
  if (g > 2048) g = 2048;
  hipLaunchKernelGGL(lora_proj_finalize_kernel, dim3((unsigned)g), dim3(256), 0, s, j0, jb,
                     njobs, M, r, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_grad: grid ((ldg0 / 64 + ldg1 / 64) * splits), 256 threads.  A block
// owns 64 columns g of the big operand G (dy for dB, x for dA), all r
// columns of the small operand S (in chunks of 16 JT) and the z-th share of the
// tokens.  Wave w takes the 32-token steps w, w + 4, ... of that share.  G
// is token-major, so the wave stores each step's G rows transposed (tokens
// contiguous) in its own LDS tile and reads 16-byte MFMA operands back; S
// comes from the transposed copy ST [2r][Mp] as direct 16-byte loads.
// 16x16x32 MFMA with G columns as rows and S columns as columns; hi and lo
// are two MFMAs on the same G operand.  No barrier is needed inside the
// loop: a wave's LDS accesses are executed in order and no other wave
// touches its tile.  With one split the block writes C itself; otherwise it
// writes the partial Cp[z] (C's layout) and lora_grad_finalize adds them in
// order.
// ---------------------------------------------------------------------------
constexpr int kGradRow = 40;               // LDS row: 32 tokens + 8 pad (bf16), 80 bytes
constexpr int kGradTile = 64 * kGradRow;   // one wave's transposed G step
constexpr int kGradRed = 68;               // fp32 row stride of the cross-wave reduction

// JT: 16-column groups of S held per step (1, 2 or 4), so small ranks keep
// few registers and more blocks fit on a CU.
template <int JT>
__global__ __launch_bounds__(256) void lora_grad_kernel(LoraGradJob j0, LoraGradJob j1,
                                                        int64_t blocks0, int64_t M, int r,
                                                        int accumulate, int splits) {
  __shared__ __align__(16) float red[4 * 64 * kGradRed];  // 69632 B; the tiles alias its start
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraGradJob J = second ? j1 : j0;
  const int64_t ldg = J.ldg;
  const int64_t bb = second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
  const int z = (int)(bb % splits);
  const int64_t g0 = 64 * (bb / splits);
  float* C = splits == 1 ? J.C : J.Cp + (int64_t)z * ldg * r;
  const int acc_out = splits == 1 ? accumulate : 0;

  uint16_t* tile = reinterpret_cast<uint16_t*>(red) + wave * kGradTile;
  const int tk = lane & 31, ch = lane >> 5;  // token of a step, chunk parity
  const int i = lane & 15, kg = lane >> 4;   // MFMA operand lane coordinates
  const int64_t Mp = pad32(M);
  const int64_t nst = Mp / 32;
  const int64_t st0 = nst * z / splits, st1 = nst * (z + 1) / splits;
  const int64_t ns = st1 - st0 > wave ? (st1 - st0 - wave + 3) / 4 : 0;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int jc = 0; jc < r; jc += 16 * JT) {
    const int R = r - jc < 16 * JT ? r - jc : 16 * JT;  // multiple of 8

    // step s of this wave: tokens t0 + tk with t0 = 32 (st0 + wave + 4 s);
    // G chunk c = ch + 2u (8 columns); S operands of the 16-column groups
    auto load_step = [&](int64_t s, u32x4_t (&gv)[4], u32x4_t (&sh)[JT], u32x4_t (&sl)[JT]) {
      const int64_t t0 = 32 * (st0 + wave + 4 * s);
      const int64_t m = t0 + tk;
      const bool ok = m < M;
      const uint16_t* grow = J.G + (ok ? m : 0) * ldg + g0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        gv[u] = ok ? *reinterpret_cast<const u32x4_t*>(grow + 8 * (ch + 2 * u)) : zero;
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        if (16 * jt < R) {
          const int col = jc + 16 * jt + i;
          const bool cok = col < r;
          const int64_t off = t0 + 8 * kg;
          sh[jt] = cok ? *reinterpret_cast<const u32x4_t*>(J.ST + (int64_t)col * Mp + off) : zero;
          sl[jt] = cok ? *reinterpret_cast<const u32x4_t*>(J.ST + (int64_t)(r + col) * Mp + off)
                       : zero;
        } else {
          sh[jt] = zero;
          sl[jt] = zero;
        }
      }
    };
    f32x4_t acc[4][JT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < JT; ++b) acc[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto mma_step = [&](const u32x4_t (&gv)[4], const u32x4_t (&sh)[JT], const u32x4_t (&sl)[JT]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tile[(8 * (ch + 2 * u) + e) * kGradRow + tk] = (uint16_t)(gv[u][e >> 1] >> (16 * (e & 1)));
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(tile + (16 * gi + i) * kGradRow + 8 * kg);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          if (16 * jt < R) {
            acc[gi][jt] = mfma16x16x32(a, sh[jt], acc[gi][jt]);
            acc[gi][jt] = mfma16x16x32(a, sl[jt], acc[gi][jt]);
          }
        }
      }
    };

    u32x4_t G0[4], H0[JT], L0[JT], G1[4], H1[JT], L1[JT];
    if (ns > 0) load_step(0, G0, H0, L0);
    for (int64_t s = 0; s < ns; s += 2) {
      if (s + 1 < ns) load_step(s + 1, G1, H1, L1);
      mma_step(G0, H0, L0);
      if (s + 1 < ns) {
        if (s + 2 < ns) load_step(s + 2, G0, H0, L0);
        mma_step(G1, H1, L1);
      }
    }

    __syncthreads();  // every wave is done with its tile; reuse LDS for the sums
    // D[g][j]: lane holds column j = lane % 16, rows 4 (lane / 16) + v
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
        if (16 * jt < R)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(wave * 64 + 16 * gi + 4 * kg + v) * kGradRed + 16 * jt + i] = acc[gi][jt][v];
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * R; e += 256) {
      // consecutive threads write consecutive addresses of C
      const int gl = J.transposed ? (e & 63) : e / R;
      const int j = J.transposed ? (e >> 6) : e % R;
      const float sum = ((red[(0 * 64 + gl) * kGradRed + j] + red[(1 * 64 + gl) * kGradRed + j]) +
                         red[(2 * 64 + gl) * kGradRed + j]) +
                        red[(3 * 64 + gl) * kGradRed + j];
      const int64_t g = g0 + gl;
      const int jo = jc + j;
      float* c = J.transposed ? C + (int64_t)jo * ldg + g : C + g * r + jo;
      *c = acc_out ? *c + sum : sum;
    }
    __syncthreads();  // before the next chunk overwrites the tiles
  }
}

// C (+)= sum_z Cp[z] (z in order), grid-stride over both jobs' outputs
__global__ __launch_bounds__(256) void lora_grad_finalize_kernel(LoraGradJob j0, LoraGradJob j1,
                                                                 int r, int accumulate,
                                                                 int splits) {
  const int64_t n0 = j0.ldg * r, total = n0 + j1.ldg * r;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const bool second = e >= n0;
    const float* Cp = second ? j1.Cp : j0.Cp;
    float* C = second ? j1.C : j0.C;
    const int64_t n = second ? total - n0 : n0;
    const int64_t ee = second ? e - n0 : e;
    float v[16];
#pragma unroll
    for (int z = 0; z < 16; ++z) v[z] = z < splits ? Cp[(int64_t)z * n + ee] : 0.0f;
    float sum = v[0];
#pragma unroll
    for (int z = 1; z < 16; ++z)
      if (z < splits) sum += v[z];
    C[ee] = accumulate ? C[ee] + sum : sum;
  }
}

int lora_grad_splits(int64_t M, int64_t ldg0, int64_t ldg1) {
  const int64_t blocks = ldg0 / 64 + ldg1 / 64;
  const int64_t nst = pad32(M) / 32;
  int64_t s = blocks > 0 ? (512 + blocks - 1) / blocks : 1;
  if (s > nst / 4) s = nst / 4;  // at least one 32-token step per wave
  if (s > kGradMaxSplits) s = kGradMaxSplits;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_lora_grad(const LoraGradJob& j0, const LoraGradJob& j1, int64_t M, int r,
                            int accumulate, int splits, hipStream_t s) {
  const int64_t b0 = j0.ldg / 64, b1 = j1.ldg / 64;
  if (b0 + b1 == 0 || r == 0) return hipSuccess;
  const dim3 grid((unsigned)((b0 + b1) * splits));
  if (r <= 16)
    hipLaunchKernelGGL(lora_grad_kernel<1>, grid, dim3(256), 0, s, j0, j1, b0 * splits, M, r,
                       accumulate, splits);
  else if (r <= 32)
    hipLaunchKernelGGL(lora_grad_kernel<2>, grid, dim3(256), 0, s, j0, j1, b0 * splits, M, r,
                       accumulate, splits);
  else
    hipLaunchKernelGGL(lora_grad_kernel<4>, grid, dim3(256), 0, s, j0, j1, b0 * splits, M, r,
                       accumulate, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  int64_t g = ((j0.ldg + j1.ldg) * r + 255) / 256;
  if (g > 2048) g = 2048;
  hipLaunchKernelGGL(lora_grad_finalize_kernel, dim3((unsigned)g), dim3(256), 0, s, j0, j1, r,
                     accumulate, splits);
  return hipGetLastError();
}

}  // namespace qlora
