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
// Both stream one big operand (x or dy) once and are bound by memory at
// training sizes and by latency at small ones.  Every block owns its
// outputs' whole reduction, so no partials leave the chip and no second
// kernel runs: the eight waves of a block take interleaved 32-wide steps of
// the reduction, each wave issues the global loads of a whole batch of
// steps before it uses them (so a block keeps many loads in flight), and
// the waves' sums are added in LDS in wave order.  Results are therefore
// deterministic.
//
// Where an MFMA operand needs 8 consecutive reduction indices of a matrix
// stored the other way round (B [Kred, r] in lora_proj, G [M, ldg] in
// lora_grad), the wave stores the loaded rows as they are into its own LDS
// slab and reads the operand back with ds_read_b64_tr_b16, gfx950's LDS
// transpose read: within each group of 16 lanes, lane i receives element
// i mod 4 of the 8-byte pieces addressed by lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4.  So if lane c of a group points at row R0 + c/4, columns
// C0 + 4 (c mod 4) .. + 3 of the slab, lane i receives rows R0 .. R0 + 3 of
// column C0 + i; two such reads (R0 and R0 + 4) give the 8 values.  A slab
// is private to its wave and a wave's LDS accesses complete in order, so no
// barrier is needed around it.

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int kWaves = 8;             // waves per block (both kernels)
constexpr int kThreads = 64 * kWaves;

__host__ __device__ __forceinline__ int64_t pad32(int64_t M) { return (M + 31) / 32 * 32; }

// Loads go through buffer descriptors: 32-bit lane offsets instead of 64-bit
// addresses, and a lane offset at or past the tensor's size reads zero
// (rows past M, rank columns past r, steps past a wave's share).  The
// scalar offset, which the bounds check does not see, carries only the
// wave-uniform step position.
constexpr uint32_t kOff = 0x80000000u;  // past every tensor (each is below 2 GiB)
__device__ __forceinline__ u32x4_t ldb(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff,
                                                                           (int)soff, 0));
}

// One byte through a buffer descriptor (zero past its end).
__device__ __forceinline__ uint32_t ldb8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// The keep-mask of a job, [rows, cols / 8] bytes, through a descriptor;
// `all` is ORed into every loaded byte (0xFF: the job has no mask, so
// every bit reads as kept).
struct KeepBits {
  __amdgpu_buffer_rsrc_t res;
  uint32_t all;
};
__device__ __forceinline__ KeepBits keep_bits(const uint8_t* keep, int64_t bytes) {
  KeepBits k;
  k.res = make_rsrc(keep, keep ? (uint32_t)bytes : 0u);
  k.all = keep ? 0u : 0xFFu;
  return k;
}

// The job a block works on is picked by comparing blockIdx with a kernel
// argument, which is the same for every lane, but the compiler cannot tell:
// a buffer descriptor built from a value it takes to differ between lanes
// gets a readfirstlane loop around every load.  Reading each field through
// readfirstlane states that it is uniform.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  return reinterpret_cast<T*>(uniform64(reinterpret_cast<uint64_t>(p)));
}
__device__ __forceinline__ LoraProjJob uniform_job(const LoraProjJob& j) {
  LoraProjJob u;
  u.X = uniform_ptr(j.X);
  u.Y = uniform_ptr(j.Y);
  u.out = uniform_ptr(j.out);
  u.outT = uniform_ptr(j.outT);
  u.Kred = (int64_t)uniform64((uint64_t)j.Kred);
  u.kmajor = __builtin_amdgcn_readfirstlane(j.kmajor);
  u.keep = uniform_ptr(j.keep);
  u.rng = __builtin_amdgcn_readfirstlane(j.rng);
  u.drop.k0 = __builtin_amdgcn_readfirstlane(j.drop.k0);
  u.drop.k1 = __builtin_amdgcn_readfirstlane(j.drop.k1);
  u.drop.o0 = __builtin_amdgcn_readfirstlane(j.drop.o0);
  u.drop.o1 = __builtin_amdgcn_readfirstlane(j.drop.o1);
  u.drop.t = __builtin_amdgcn_readfirstlane(j.drop.t);
  u.keep_out = uniform_ptr(j.keep_out);
  u.S = __builtin_amdgcn_readfirstlane(j.S);
  u.part = uniform_ptr(j.part);
  return u;
}
__device__ __forceinline__ LoraGradJob uniform_job(const LoraGradJob& j) {
  LoraGradJob u;
  u.G = uniform_ptr(j.G);
  u.ST = uniform_ptr(j.ST);
  u.C = uniform_ptr(j.C);
  u.ldg = (int64_t)uniform64((uint64_t)j.ldg);
  u.transposed = __builtin_amdgcn_readfirstlane(j.transposed);
  u.keep = uniform_ptr(j.keep);
  return u;
}

// 8 bf16 of one slab column: rows row0 .. row0 + 7 (as two transpose reads,
// rows row0 + 4h + c/4 addressed by lane c of the 16-lane group), column
// col0 + lane % 16.  `stride` is the slab row length in bf16.
__device__ __forceinline__ u32x4_t read_tr8(const uint16_t* slab, int stride, int row0, int col0,
                                            int i) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const uint16_t* p = slab + (row0 + (i >> 2)) * stride + col0 + 4 * (i & 3);
  const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * stride));
  const u32x2_t h0 = __builtin_bit_cast(u32x2_t, r0), h1 = __builtin_bit_cast(u32x2_t, r1);
  const u32x4_t v = {h0[0], h0[1], h1[0], h1[1]};
  return v;
}

// Store the 16-bit pair (compute type DT) of v for (m, j) in both layouts
// (m < Mp; rows past M only get zeros in the transposed copy).
template <class DT>
__device__ __forceinline__ void put_split(const LoraProjJob& J, int64_t M, int r, int64_t m,
                                          int j, float v) {
  const int64_t Mp = pad32(M);
  uint16_t hi = 0, lo = 0;
  if (m < M) {
    hi = DT::cvt(v);
    lo = DT::cvt(v - DT::tof(hi));  // v - hi is exact
    J.out[m * 2 * r + j] = hi;
    J.out[m * 2 * r + r + j] = lo;
  }
  J.outT[(int64_t)j * Mp + m] = hi;
  J.outT[(int64_t)(r + j) * Mp + m] = lo;
}

}  // namespace

// ---------------------------------------------------------------------------
// lora_proj: grid = sum over jobs of ceil(Mp / (16 TT)) * ceil(r / RC) * S
// blocks, 512 threads.  A block owns 16 TT tokens x RC = 16 JT rank columns
// of one job and a contiguous 1/S share of that job's 32-wide reduction
// steps; wave w takes the block's steps w, w + 8, ... with 16x16x32 MFMA
// (tokens as rows).  The token operand is one 16-byte load per lane and
// token tile (8 consecutive k of a row); A's operand is one per 16-column
// group, shared by the TT token tiles, so a block reads A (or B) once for
// 16 TT tokens -- at training sizes the small operand, re-read by every
// token block, is what the kernel's L2 traffic is made of.  B's rows (8
// rank columns of one k per 16 bytes) go through the wave's slab and come
// back transposed, once per step for all TT tiles.  The waves' sums are
// added in LDS in wave order, one token tile at a time; with S = 1 the
// block stores the hi/lo pairs itself, otherwise fp32 partials that
// lora_proj_finalize adds in split order.
// ---------------------------------------------------------------------------
// DROP: LoRA dropout on X (see keep8): 0 none, 1 the jobs may carry a
// keep-mask, 2 a job may draw its keep bits (rng) -- the blocks of the first
// rank chunk then also store them to keep_out.
template <int JT, int TT, int DROP, class DT>
__global__ __launch_bounds__(kThreads) void lora_proj_kernel(LoraProjJob j0, LoraProjJob j1,
                                                             int64_t blocks0, int64_t M, int r,
                                                             float scale) {
  constexpr int RC = 16 * JT;            // rank columns of the block
  constexpr int RS = RC + 8;             // slab row: RC bf16 + 16 bytes of pad
  constexpr int SLAB = 32 * RS;          // bf16 per wave
  // k steps per batch of loads (a batch holds TT + JT operands per step;
  // sized so that no variant spills)
  constexpr int BS = TT >= 4 ? (TT == 4 && DROP == 0 ? 2 : 1) : (TT == 2 ? 2 : (JT == 1 ? 8 : (JT == 2 ? 4 : 2)));
  constexpr int REDS = RC + 4;           // fp32 row of the cross-wave sums
  constexpr int SLAB_BYTES = kWaves * SLAB * 2, RED_BYTES = kWaves * 16 * REDS * 4;
  __shared__ __align__(16) char lds[SLAB_BYTES > RED_BYTES ? SLAB_BYTES : RED_BYTES];

  const int t = threadIdx.x, lane = t & 63;
  // the wave index, stated uniform (scalar offsets are built from it)
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraProjJob J = uniform_job(second ? j1 : j0);
  const int64_t b = second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
  const int jchunks = (r + RC - 1) / RC;
  const int S = J.S;
  const int z = (int)(b % S);
  const int64_t rest = b / S;
  const int64_t m0 = 16 * TT * (rest / jchunks);
  const int jc = (int)(rest % jchunks) * RC;
  const int i = lane & 15, kg = lane >> 4;
  const int64_t Kred = J.Kred;
  const int64_t nsteps = Kred / 32;
  const int64_t s0 = nsteps * z / S, s1 = nsteps * (z + 1) / S;
  const int64_t cnt = s1 - s0 > wave ? (s1 - s0 - wave + kWaves - 1) / kWaves : 0;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(J.X, (uint32_t)(M * Kred * 2));
  const __amdgpu_buffer_rsrc_t yres = make_rsrc(J.Y, (uint32_t)((int64_t)r * Kred * 2));
  // rows m in [M, Mp) (and past Mp) lie past x's end and read as zero
  uint32_t xoff[TT], koff[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int64_t m = m0 + 16 * tt + i;
    xoff[tt] = (uint32_t)((m * Kred + 8 * kg) * 2);
    koff[tt] = (uint32_t)(m * (Kred / 8) + kg);  // keep byte of the lane's x chunk: + k0 / 8
  }
  uint16_t* slab = reinterpret_cast<uint16_t*>(lds) + wave * SLAB;
  const bool kmajor = J.kmajor != 0;
  const KeepBits kp = keep_bits(J.keep, M * Kred / 8);

  f32x4_t acc[TT][JT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[tt][jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Y pieces of a step: A: column group jt's 16 bytes; B: piece p = lane +
  // 64 q of the 32 x RC slab, row p / (2 JT), 8 columns at 8 (p mod 2 JT)
  struct Batch {
    u32x4_t x[BS][TT];
    u32x4_t y[BS][JT];
    uint32_t kb[BS][TT];
  };
  // Lane offsets of the Y pieces, fixed for the whole loop (kOff past r).
  // Steps past the wave's count OR in kOff: a select the compiler keeps as
  // one (a branch around the loads would make it wait for each load).
  uint32_t yoff[JT];
#pragma unroll
  for (int q = 0; q < JT; ++q) {
    if (!kmajor) {
      const int jj = jc + 16 * q + i;
      yoff[q] = jj < r ? (uint32_t)jj * (uint32_t)Kred * 2u + 16u * (uint32_t)kg : kOff;
    } else {
      const int p = lane + 64 * q, row = p / (2 * JT), col = jc + 8 * (p % (2 * JT));
      yoff[q] = col < r ? (uint32_t)(row * r + col) * 2u : kOff;
    }
  }
  auto k_of = [&](int64_t u) { return (uint32_t)(32 * (s0 + wave + kWaves * u)); };
  auto load = [&](int64_t u0, Batch& R) {
#pragma unroll
    for (int bb = 0; bb < BS; ++bb) {
      const int64_t u = u0 + bb;
      const uint32_t past = u < cnt ? 0u : kOff;
      const uint32_t k0 = k_of(u);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        R.x[bb][tt] = ldb(xres, xoff[tt] | past, 2 * k0);
        if constexpr (DROP == 1) R.kb[bb][tt] = ldb8(kp.res, koff[tt] | past, k0 / 8) | kp.all;
      }
#pragma unroll
      for (int q = 0; q < JT; ++q)
        R.y[bb][q] = ldb(yres, yoff[q] | past, kmajor ? 2 * k0 * (uint32_t)r : 2 * k0);
    }
  };
  // drawn keep bytes: the first rank chunk's blocks store those of real
  // tokens and steps
  const bool store_keep = DROP == 2 && J.keep_out != nullptr && jc == 0;
  // steps past the wave's count carry zero operands and add nothing
  auto compute = [&](const Batch& R, int64_t u0) {
#pragma unroll
    for (int bb = 0; bb < BS; ++bb) {
      const int64_t u = u0 + bb;
      if (kmajor) {
#pragma unroll
        for (int q = 0; q < JT; ++q) {
          const int p = lane + 64 * q, row = p / (2 * JT), cp = p % (2 * JT);
          *reinterpret_cast<u32x4_t*>(slab + row * RS + 8 * cp) = R.y[bb][q];
        }
      }
      // B's operands from the slab: read each once for the TT tiles (with
      // one tile, one at a time next to its MFMA, which keeps fewer live)
      u32x4_t yv[JT];
      if constexpr (TT > 1) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
          yv[jt] = kmajor ? read_tr8(slab, RS, 8 * kg, 16 * jt, i) : R.y[bb][jt];
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        uint32_t kb = 0xFFu;
        if constexpr (DROP == 1) kb = R.kb[bb][tt];
        if constexpr (DROP == 2) {
          if (J.rng) {
            const uint32_t chunk = koff[tt] + k_of(u) / 8;
            kb = philox_keep_byte(J.drop, chunk);
            if (store_keep && u < cnt && m0 + 16 * tt + i < M) J.keep_out[chunk] = (uint8_t)kb;
          }
        }
        const u32x4_t xv = DROP ? keep8(R.x[bb][tt], kb) : R.x[bb][tt];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          if constexpr (TT > 1)
            acc[tt][jt] = DT::mfma16(xv, yv[jt], acc[tt][jt]);
          else
            acc[tt][jt] = DT::mfma16(
                xv, kmajor ? read_tr8(slab, RS, 8 * kg, 16 * jt, i) : R.y[bb][jt], acc[tt][jt]);
        }
      }
    }
  };

  // Loads are unconditional (steps past the count read zeros, which add
  // nothing): a branch around them would make the compiler, at the join,
  // wait for the newer batch too before computing the older one.  The
  // fences keep each batch's loads ahead of the compute before them.
  Batch R0, R1;
  load(0, R0);
  for (int64_t u0 = 0; u0 < cnt; u0 += 2 * BS) {
    load(u0 + BS, R1);
    __builtin_amdgcn_sched_barrier(0);
    compute(R0, u0);
    load(u0 + 2 * BS, R0);
    __builtin_amdgcn_sched_barrier(0);
    compute(R1, u0 + BS);
  }

  // D[token][j]: lane holds column j = 16 jt + lane % 16, tokens 4 (lane / 16) + v
  float* red = reinterpret_cast<float*>(lds);
  const int64_t Mp = pad32(M);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    __syncthreads();  // every slab (first tile) or the last tile's sums are done
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(wave * 16 + 4 * kg + v) * REDS + 16 * jt + i] = acc[tt][jt][v];
    __syncthreads();
    for (int e = t; e < 16 * RC; e += kThreads) {
      const int tok = e & 15, j = e >> 4;  // tokens fastest: outT rows are token-contiguous
      float sum = red[tok * REDS + j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) sum += red[(w * 16 + tok) * REDS + j];
      const int64_t mo = m0 + 16 * tt + tok;
      const int jo = jc + j;
      if (jo < r && mo < Mp) {
        if (S == 1)
          put_split<DT>(J, M, r, mo, jo, scale * sum);
        else
          J.part[((int64_t)z * r + jo) * Mp + mo] = sum;
      }
    }
  }
}

// The split jobs' hi/lo pairs: element e of a job is (j, m) = (e / Mp,
// e % Mp); its S partials are added in split order and scaled once.
template <class DT>
__global__ __launch_bounds__(256) void lora_proj_finalize_kernel(LoraProjJob j0, LoraProjJob j1,
                                                                 int64_t n0, int64_t M, int r,
                                                                 float scale) {
  const int64_t Mp = pad32(M);
  int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = e >= n0;
  const LoraProjJob& J = second ? j1 : j0;
  if (second) e -= n0;
  if (e >= Mp * r) return;
  const int j = (int)(e / Mp);
  const int64_t m = e % Mp;
  float sum = 0.0f;
  for (int zz = 0; zz < J.S; ++zz) sum += J.part[((int64_t)zz * r + j) * Mp + m];
  put_split<DT>(J, M, r, m, j, scale * sum);
}

// ---------------------------------------------------------------------------
// lora_proj_small: the same product when M r is small (few tokens and a
// small rank).  With 16 x 16 MFMA tiles such a job has only M / 16 blocks,
// and each has to pull in a whole 16-row slice of x plus all of Y; here a
// block owns TT tokens x 8 rank columns (so M r / (8 TT) blocks, each
// reading TT + 8 rows) and the whole reduction: TT = 8, or 4 when 8-token
// blocks would leave CUs without one.  Its 256 threads take the 8-wide pieces
// of the reduction t, t + 256, ... and accumulate with v_dot2_f32_bf16
// (two bf16 products added into an fp32 sum, no conversions).  B's pieces
// (8 rank columns of one k) are turned into (k, k + 1) pairs of one column
// with one v_perm per pair.  The 256 threads' sums are added in LDS in a
// fixed order, then by a fixed butterfly over 256 / (8 TT) lanes.
// ---------------------------------------------------------------------------
constexpr int kSmallR = 8;     // rank columns per block
constexpr int kSmallRed = 65;  // LDS row of a thread's (up to) 64 sums (+1: no bank conflicts)

template <int DROP, class DT, int TT>
__global__ __launch_bounds__(256) void lora_proj_small_kernel(LoraProjJob j0, LoraProjJob j1,
                                                              int64_t blocks0, int64_t M, int r,
                                                              float scale) {
  __shared__ float red[256 * kSmallRed];
  const int t = threadIdx.x;
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraProjJob J = uniform_job(second ? j1 : j0);
  const int64_t b = second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x;
  const int rg = r / kSmallR;
  const int64_t m0 = TT * (b / rg);
  const int jc = (int)(b % rg) * kSmallR;
  const int64_t Kred = J.Kred;
  const int64_t npc = Kred / 8;  // 8-wide pieces of the reduction
  const int64_t cnt = npc > t ? (npc - t + 255) / 256 : 0;
  const bool kmajor = J.kmajor != 0;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(J.X, (uint32_t)(M * Kred * 2));
  const __amdgpu_buffer_rsrc_t yres = make_rsrc(J.Y, (uint32_t)((int64_t)r * Kred * 2));
  // rows past M lie past x's end and read as zero
  uint32_t xoff[TT], koff[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    xoff[i] = (uint32_t)((m0 + i) * Kred * 2);
    koff[i] = (uint32_t)((m0 + i) * (Kred / 8));  // keep byte of piece pc: koff + pc
  }
  const KeepBits kp = keep_bits(J.keep, M * Kred / 8);

  float acc[TT][kSmallR];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < kSmallR; ++j) acc[i][j] = 0.0f;

  // piece u of this thread: k = 8 (t + 256 u) .. + 7; x rows, then Y: A's
  // rows jc .. jc + 7 (kmajor == 0) or B's rows k .. k + 7 (kmajor == 1)
  struct Piece {
    u32x4_t x[TT];
    u32x4_t y[kSmallR];
    uint32_t kb[TT];
  };
  // Every offset here differs between lanes, so all of it is lane offset.
  // Pieces past the thread's count OR in kOff: a select the compiler keeps
  // as one (a branch around the loads would make it wait for each load).
  uint32_t ybase[kSmallR];
#pragma unroll
  for (int q = 0; q < kSmallR; ++q)
    ybase[q] = kmajor ? (uint32_t)(q * r + jc) * 2u : (uint32_t)(jc + q) * (uint32_t)Kred * 2u;
  auto load = [&](int64_t u, Piece& P) {
    const uint32_t past = u < cnt ? 0u : kOff;
    const uint32_t pc = (uint32_t)(t + 256 * u);  // 8-wide piece index
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      P.x[i] = ldb(xres, (xoff[i] + 16u * pc) | past, 0);
      if constexpr (DROP == 1) P.kb[i] = ldb8(kp.res, (koff[i] + pc) | past, 0) | kp.all;
    }
#pragma unroll
    for (int q = 0; q < kSmallR; ++q)
      P.y[q] = ldb(yres, (ybase[q] + (kmajor ? 16u * (uint32_t)r * pc : 16u * pc)) | past, 0);
  };

  // drawn keep bytes: the first rank group's blocks store those of real
  // tokens and pieces
  const bool store_keep = DROP == 2 && J.keep_out != nullptr && jc == 0;
  auto compute = [&](const Piece& P, int64_t u) {
    u32x4_t yp[kSmallR];  // column q's (k, k + 1) pairs
#pragma unroll
    for (int q = 0; q < kSmallR; ++q) {
      if (!kmajor) {
        yp[q] = P.y[q];
      } else {
        // column q sits in dword q / 2 of each B row piece, half q % 2
        const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          yp[q][pp] = perm(P.y[2 * pp + 1][q >> 1], P.y[2 * pp][q >> 1], sel);
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      uint32_t kb = 0xFFu;
      if constexpr (DROP == 1) kb = P.kb[i];
      if constexpr (DROP == 2) {
        if (J.rng) {
          const uint32_t chunk = koff[i] + (uint32_t)(t + 256 * u);
          kb = philox_keep_byte(J.drop, chunk);
          if (store_keep && u < cnt && m0 + i < M) J.keep_out[chunk] = (uint8_t)kb;
        }
      }
      const u32x4_t xv = DROP ? keep8(P.x[i], kb) : P.x[i];
#pragma unroll
      for (int q = 0; q < kSmallR; ++q)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          acc[i][q] = DT::dot2(xv[pp], yp[q][pp], acc[i][q]);
    }
  };
  // Loads are unconditional (a piece past the count reads zeros, which add
  // nothing): a branch around them would leave the compiler, at the join,
  // waiting for the newer piece as well before computing the older one.
  // The fences keep each piece's loads ahead of the compute before them
  // (the scheduler otherwise sinks them below it).
  Piece P0, P1;
  load(0, P0);
  for (int64_t u = 0; u < cnt; u += 2) {
    load(u + 1, P1);
    __builtin_amdgcn_sched_barrier(0);
    compute(P0, u);
    load(u + 2, P0);
    __builtin_amdgcn_sched_barrier(0);
    compute(P1, u + 1);
  }

#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int q = 0; q < kSmallR; ++q) red[t * kSmallRed + i * kSmallR + q] = acc[i][q];
  __syncthreads();
  // output o = t / LPO (TT x 8 outputs): its 256 sums, lane t % LPO taking
  // every LPO-th, then a butterfly over those LPO lanes.  The trip count is
  // a constant so the loop unrolls and its LDS reads are issued together (a
  // lane-dependent bound left one read and one wait per step).
  constexpr int LPO = 256 / (TT * kSmallR);
  const int o = t / LPO, part = t % LPO;
  float sum = red[part * kSmallRed + o];
#pragma unroll
  for (int i = 1; i < 256 / LPO; ++i) sum += red[(part + LPO * i) * kSmallRed + o];
#pragma unroll
  for (int w = 1; w < LPO; w <<= 1) sum += __shfl_xor(sum, w, LPO);
  const int64_t Mp = pad32(M);
  const int64_t mo = m0 + o / kSmallR;
  const int jo = jc + o % kSmallR;
  if (part == 0 && mo < Mp && jo < r) put_split<DT>(J, M, r, mo, jo, scale * sum);
}

// small jobs (few tokens x a small rank) go to lora_proj_small: measured
// faster at q_proj (M = 512, r = 16), slower at M = 2048, r = 16
static bool proj_small(int64_t M, int r) { return M * r <= 16384; }

static int proj_jt(int r) { return r <= 16 ? 1 : (r <= 32 ? 2 : 4); }

// Token tiles per block: the largest (up to 8, or 4 for ranks above 32)
// that leaves at least 16 token blocks.  Splits: about 256 blocks in all, dealt to the jobs in
// proportion to their reduction lengths, each split at least two steps per
// wave and at most 16 splits.
ProjPlan lora_proj_plan(int64_t M, int r, int64_t kred0, int64_t kred1) {
  ProjPlan p{};
  p.s[0] = p.s[1] = 1;
  p.tt = 1;
  if (r == 0 || M == 0) return p;
  if (proj_small(M, r)) {
    p.small = true;
    return p;
  }
  const int64_t Mp = pad32(M);
  const int rc = 16 * proj_jt(r);
  const int64_t jch = (r + rc - 1) / rc;
  // (at most 4 with rank tiles of 64 columns: 8 would not fit the registers)
  int tt = proj_jt(r) == 4 ? 4 : 8;
  while (tt > 1 && Mp / (16 * tt) < 16) tt /= 2;
  p.tt = tt;
  const int64_t base = (Mp + 16 * tt - 1) / (16 * tt) * jch;  // blocks per job, unsplit
  const int64_t ktot = kred0 + kred1;
  for (int j = 0; j < 2; ++j) {
    const int64_t kr = j ? kred1 : kred0;
    if (kr <= 0) continue;
    int64_t sj = (256 * kr + ktot * base / 2) / (ktot * base);
    const int64_t smax = kr / (32 * kWaves * 2);
    if (sj > smax) sj = smax;
    if (sj > 16) sj = 16;
    if (sj < 1) sj = 1;
    p.s[j] = (int)sj;
  }
  return p;
}

size_t lora_proj_partial_bytes(const ProjPlan& p, int job, int64_t M, int r) {
  if (p.small || p.s[job] <= 1) return 0;
  return (size_t)p.s[job] * (size_t)r * (size_t)pad32(M) * sizeof(float);
}

template <int JT, int TT, int DROP, class DT>
static void launch_proj_tiled(dim3 grid, hipStream_t s, const LoraProjJob& j0,
                              const LoraProjJob& jb, int64_t blocks0, int64_t M, int r,
                              float scale) {
  hipLaunchKernelGGL((lora_proj_kernel<JT, TT, DROP, DT>), grid, dim3(kThreads), 0, s, j0, jb,
                     blocks0, M, r, scale);
}

template <int JT, int DROP, class DT>
static void launch_proj_tt(int tt, dim3 grid, hipStream_t s, const LoraProjJob& j0,
                           const LoraProjJob& jb, int64_t blocks0, int64_t M, int r,
                           float scale) {
  if constexpr (JT < 4) {
    if (tt >= 8) {
      launch_proj_tiled<JT, 8, DROP, DT>(grid, s, j0, jb, blocks0, M, r, scale);
      return;
    }
  }
  if (tt >= 4)
    launch_proj_tiled<JT, 4, DROP, DT>(grid, s, j0, jb, blocks0, M, r, scale);
  else if (tt == 2)
    launch_proj_tiled<JT, 2, DROP, DT>(grid, s, j0, jb, blocks0, M, r, scale);
  else
    launch_proj_tiled<JT, 1, DROP, DT>(grid, s, j0, jb, blocks0, M, r, scale);
}

template <int DROP, class DT>
static hipError_t launch_proj(const LoraProjJob& j0, const LoraProjJob* j1, int64_t M, int r,
                              float scale, hipStream_t s) {
  const ProjPlan plan = lora_proj_plan(M, r, j0.Kred, j1 ? j1->Kred : 0);
  if (plan.small) {
    // Mp / TT token groups cover every row of the transposed copy; 4-token
    // blocks when 8-token ones would not give every CU a block
    const int jobs = j1 ? 2 : 1;
    const bool t4 = (pad32(M) / 8) * (r / kSmallR) * jobs < 256;
    const int64_t per_job = (pad32(M) / (t4 ? 4 : 8)) * (r / kSmallR);
    const LoraProjJob jb = j1 ? *j1 : j0;
    const int64_t total = per_job * jobs;
    if (total == 0) return hipSuccess;
    if (t4)
      hipLaunchKernelGGL((lora_proj_small_kernel<DROP, DT, 4>), dim3((unsigned)total), dim3(256),
                         0, s, j0, jb, per_job, M, r, scale);
    else
      hipLaunchKernelGGL((lora_proj_small_kernel<DROP, DT, 8>), dim3((unsigned)total), dim3(256),
                         0, s, j0, jb, per_job, M, r, scale);
    return hipGetLastError();
  }
  const int jt = proj_jt(r);
  const int rc = 16 * jt;
  LoraProjJob a = j0, b = j1 ? *j1 : j0;
  a.S = plan.s[0];
  b.S = j1 ? plan.s[1] : plan.s[0];
  if ((a.S > 1 && !a.part) || (j1 && b.S > 1 && !b.part)) return hipErrorInvalidValue;
  // ceil(Mp / (16 TT)) token blocks cover every row of the transposed copy
  const int64_t tiles = (pad32(M) + 16 * plan.tt - 1) / (16 * plan.tt) * ((r + rc - 1) / rc);
  const int64_t blocks0 = tiles * a.S, total = blocks0 + (j1 ? tiles * b.S : 0);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)total);
  if (jt == 1)
    launch_proj_tt<1, DROP, DT>(plan.tt, grid, s, a, b, blocks0, M, r, scale);
  else if (jt == 2)
    launch_proj_tt<2, DROP, DT>(plan.tt, grid, s, a, b, blocks0, M, r, scale);
  else
    launch_proj_tt<4, DROP, DT>(plan.tt, grid, s, a, b, blocks0, M, r, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n0 = a.S > 1 ? pad32(M) * r : 0;
  const int64_t n1 = (j1 && b.S > 1) ? pad32(M) * r : 0;
  if (n0 + n1 == 0) return hipSuccess;
  // a job that is not split already stored its pairs: give the finalize
  // only the split ones (an unsplit first job is replaced by the second)
  const LoraProjJob& f0 = n0 ? a : b;
  hipLaunchKernelGGL((lora_proj_finalize_kernel<DT>), dim3((unsigned)((n0 + n1 + 255) / 256)),
                     dim3(256), 0, s, f0, b, n0 ? n0 : n1, M, r, scale);
  return hipGetLastError();
}

hipError_t launch_lora_proj(const LoraProjJob& j0, const LoraProjJob* j1, int64_t M, int r,
                            float scale, hipStream_t s, bool f16) {
  if (f16) return launch_proj<0, F16T>(j0, j1, M, r, scale, s);  // no dropout in fp16
  if (j0.rng || (j1 && j1->rng)) return launch_proj<2, Bf16T>(j0, j1, M, r, scale, s);
  if (j0.keep || (j1 && j1->keep)) return launch_proj<1, Bf16T>(j0, j1, M, r, scale, s);
  return launch_proj<0, Bf16T>(j0, j1, M, r, scale, s);
}

// The packed keep mask [M, K / 8] of a drawn dropout: one byte per thread.
__global__ __launch_bounds__(256) void dropout_mask_kernel(PhiloxDrop drop, int64_t nbytes,
                                                           uint8_t* keep) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b < nbytes) keep[b] = (uint8_t)philox_keep_byte(drop, (uint32_t)b);
}

hipError_t launch_dropout_mask(const PhiloxDrop& drop, int64_t M, int64_t K, uint8_t* keep,
                               hipStream_t s) {
  const int64_t nbytes = M * (K / 8);
  if (nbytes == 0) return hipSuccess;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((nbytes + 255) / 256)), dim3(256), 0,
                     s, drop, nbytes, keep);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_grad: grid = (ldg0 + ldg1) / CT blocks, 512 threads.  A block owns CT
// = 64 CW columns g0 .. g0 + CT - 1 of the big operand G (dy for dB, x for
// dA), all r columns of the small operand S (in chunks of RC = 16 JT) and
// every token.  Wave w takes the 32-token steps w, w + 8, ...: it stores the
// step's G rows (tokens x CT columns, as loaded) in its slab and reads
// 16 x 32 MFMA operands back transposed (G columns as rows, 8 consecutive
// tokens per lane); S comes from the transposed copy ST [2r][Mp] as direct
// 16-byte loads, hi and lo as two MFMAs on the same G operand.  A load of G
// covers 8 / CW token rows x 128 CW contiguous bytes: with CW = 2 the runs
// of 256 bytes per row stream from HBM markedly faster than runs of 128
// (taken when the jobs' columns fill most CUs with the wider tiles).
// ---------------------------------------------------------------------------
// DROP: the jobs may carry a keep-mask on G (LoRA dropout; see keep8).
template <int JT, bool DROP, class DT, int CW>
__global__ __launch_bounds__(64 * (CW == 1 ? kWaves : 4)) void lora_grad_kernel(LoraGradJob j0, LoraGradJob j1,
                                                             int64_t blocks0, int64_t M, int r,
                                                             int accumulate) {
  constexpr int RC = 16 * JT;
  constexpr int CT = 64 * CW;                       // G columns of the block
  // waves per block: 8, or 4 with the wide tile (one per SIMD: its
  // accumulators and two steps of loads need the whole register file)
  constexpr int NW = CW == 1 ? kWaves : 4;
  constexpr int NQ = 4 * CW;                        // G loads per step (and 16-column tiles)
  // slab row: CT bf16 + pad; row strides of 36 dwords mod 64 banks keep the
  // transposed reads conflict-free
  constexpr int GS = CW == 1 ? 64 + 8 : CT + 72;
  constexpr int SLAB = 32 * GS;                     // bf16 per wave
  // token steps per batch of loads (one with a keep-mask: its bytes would
  // otherwise push the r <= 32 variant past its registers)
  constexpr int BS = (JT == 4 || DROP) ? 1 : 2;
  constexpr int REDS = RC + 4;
  constexpr int SLAB_BYTES = NW * SLAB * 2, RED_BYTES = NW * 16 * REDS * 4;
  __shared__ __align__(16) char lds[SLAB_BYTES > RED_BYTES ? SLAB_BYTES : RED_BYTES];

  const int t = threadIdx.x, lane = t & 63;
  // the wave index, stated uniform (scalar offsets are built from it)
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraGradJob J = uniform_job(second ? j1 : j0);
  const int64_t ldg = J.ldg;
  const int64_t g0 = CT * (second ? (int64_t)blockIdx.x - blocks0 : (int64_t)blockIdx.x);
  const int i = lane & 15, kg = lane >> 4;
  const int64_t Mp = pad32(M);
  const int64_t nst = Mp / 32;
  const int64_t cnt = nst > wave ? (nst - wave + NW - 1) / NW : 0;
  uint16_t* slab = reinterpret_cast<uint16_t*>(lds) + wave * SLAB;
  float* red = reinterpret_cast<float*>(lds);
  const __amdgpu_buffer_rsrc_t gres = make_rsrc(J.G, (uint32_t)(M * ldg * 2));
  const __amdgpu_buffer_rsrc_t sres = make_rsrc(J.ST, (uint32_t)(2 * r * Mp * 2));
  const uint32_t sl_off = (uint32_t)(r * Mp * 2);  // lo rows follow the hi rows
  const KeepBits kp = keep_bits(J.keep, M * ldg / 8);

  for (int jc = 0; jc < r; jc += RC) {
    f32x4_t acc[NQ][JT];
#pragma unroll
    for (int a = 0; a < NQ; ++a)
#pragma unroll
      for (int b = 0; b < JT; ++b) acc[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // G piece p = lane + 64 q of a step: token p / (8 CW), 8 columns at
    // 8 (p mod 8 CW)
    uint32_t goff[NQ], kgoff[NQ], soff[JT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int p = lane + 64 * q, tk = p / (8 * CW), pc = p % (8 * CW);
      goff[q] = (uint32_t)(((tk * ldg) + g0 + 8 * pc) * 2);
      kgoff[q] = (uint32_t)(tk * (ldg / 8) + g0 / 8 + pc);  // the piece's keep byte
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
      soff[jt] = (uint32_t)(((int64_t)(jc + 16 * jt + i) * Mp + 8 * kg) * 2);
    struct Batch {
      u32x4_t g[BS][NQ];
      u32x4_t sh[BS][JT], sl[BS][JT];
      uint32_t kb[BS][NQ];
    };
    auto load = [&](int64_t u0, Batch& R) {
#pragma unroll
      for (int bb = 0; bb < BS; ++bb) {
        const int64_t u = u0 + bb;
        const bool ok = u < cnt;
        const uint32_t t0 = (uint32_t)(32 * (wave + NW * u));
        // the G row is part of the lane offset (rows past M read as zero)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          R.g[bb][q] = ldb(gres, ok ? goff[q] + t0 * (uint32_t)ldg * 2 : kOff, 0);
          if constexpr (DROP)
            R.kb[bb][q] = ldb8(kp.res, ok ? kgoff[q] + t0 * (uint32_t)(ldg / 8) : kOff, 0) | kp.all;
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          const bool cok = ok && jc + 16 * jt + i < r;
          R.sh[bb][jt] = ldb(sres, cok ? soff[jt] : kOff, 2 * t0);
          R.sl[bb][jt] = ldb(sres, cok ? soff[jt] + sl_off : kOff, 2 * t0);
        }
      }
    };
    auto compute = [&](const Batch& R) {
#pragma unroll
      for (int bb = 0; bb < BS; ++bb) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int p = lane + 64 * q;
          *reinterpret_cast<u32x4_t*>(slab + (p / (8 * CW)) * GS + 8 * (p % (8 * CW))) =
              DROP ? keep8(R.g[bb][q], R.kb[bb][q]) : R.g[bb][q];
        }
#pragma unroll
        for (int gi = 0; gi < NQ; ++gi) {
          const u32x4_t a = read_tr8(slab, GS, 8 * kg, 16 * gi, i);
#pragma unroll
          for (int jt = 0; jt < JT; ++jt) {
            acc[gi][jt] = DT::mfma16(a, R.sh[bb][jt], acc[gi][jt]);
            acc[gi][jt] = DT::mfma16(a, R.sl[bb][jt], acc[gi][jt]);
          }
        }
      }
    };

    // unconditional loads, as in lora_proj (zeros past the count)
    Batch R0, R1;
    load(0, R0);
    for (int64_t u0 = 0; u0 < cnt; u0 += 2 * BS) {
      load(u0 + BS, R1);
      __builtin_amdgcn_sched_barrier(0);
      compute(R0);
      load(u0 + 2 * BS, R0);
      __builtin_amdgcn_sched_barrier(0);
      compute(R1);
    }

    // D[g][j]: lane holds column j = 16 jt + lane % 16, rows 4 (lane / 16) + v
    // of G-column tile gi; one tile's wave sums at a time
    const int R = r - jc < RC ? r - jc : RC;
#pragma unroll
    for (int gi = 0; gi < NQ; ++gi) {
      __syncthreads();  // slabs (first tile) or the last tile's sums are done
#pragma unroll
      for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[(wave * 16 + 4 * kg + v) * REDS + 16 * jt + i] = acc[gi][jt][v];
      __syncthreads();
      for (int e = t; e < 16 * R; e += 64 * NW) {
        // consecutive threads write consecutive addresses of C
        const int gl = J.transposed ? (e & 15) : e / R;
        const int j = J.transposed ? (e >> 4) : e % R;
        float sum = red[gl * REDS + j];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[(w * 16 + gl) * REDS + j];
        const int64_t g = g0 + 16 * gi + gl;
        const int jo = jc + j;
        float* c = J.transposed ? J.C + (int64_t)jo * ldg + g : J.C + g * r + jo;
        *c = accumulate ? *c + sum : sum;
      }
    }
    __syncthreads();  // before the next chunk's slabs overwrite the sums
  }
}

template <bool DROP, class DT, int CW>
static void launch_grad_cw(dim3 grid, hipStream_t s, const LoraGradJob& j0,
                           const LoraGradJob& j1, int64_t b0, int64_t M, int r,
                           int accumulate) {
  const int threads = 64 * (CW == 1 ? kWaves : 4);
  if (r <= 16)
    hipLaunchKernelGGL((lora_grad_kernel<1, DROP, DT, CW>), grid, dim3(threads), 0, s, j0, j1,
                       b0, M, r, accumulate);
  else if (r <= 32)
    hipLaunchKernelGGL((lora_grad_kernel<2, DROP, DT, CW>), grid, dim3(threads), 0, s, j0, j1,
                       b0, M, r, accumulate);
  else
    hipLaunchKernelGGL((lora_grad_kernel<4, DROP, DT, CW>), grid, dim3(threads), 0, s, j0, j1,
                       b0, M, r, accumulate);
}

// 128-column tiles when both jobs' columns divide into them and they still
// give at least 224 blocks (most CUs one); 64-column ones otherwise
template <bool DROP, class DT>
static hipError_t launch_grad(const LoraGradJob& j0, const LoraGradJob& j1, int64_t M, int r,
                              int accumulate, hipStream_t s) {
  if (r == 0 || j0.ldg + j1.ldg == 0) return hipSuccess;
  const bool wide = j0.ldg % 128 == 0 && j1.ldg % 128 == 0 && (j0.ldg + j1.ldg) / 128 >= 224;
  const int ct = wide ? 128 : 64;
  const int64_t b0 = j0.ldg / ct, b1 = j1.ldg / ct;
  const dim3 grid((unsigned)(b0 + b1));
  if (wide)
    launch_grad_cw<DROP, DT, 2>(grid, s, j0, j1, b0, M, r, accumulate);
  else
    launch_grad_cw<DROP, DT, 1>(grid, s, j0, j1, b0, M, r, accumulate);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const LoraGradJob& j0, const LoraGradJob& j1, int64_t M, int r,
                            int accumulate, hipStream_t s, bool f16) {
  if (f16) return launch_grad<false, F16T>(j0, j1, M, r, accumulate, s);  // no dropout in fp16
  if (j0.keep || j1.keep) return launch_grad<true, Bf16T>(j0, j1, M, r, accumulate, s);
  return launch_grad<false, Bf16T>(j0, j1, M, r, accumulate, s);
}

}  // namespace qlora
