// Fused backward GEMM for the input gradient (gfx950):
//     dX = dy . deq(W) + (alpha/r) . (dy . B) . A
//
// [QLoRA -- the democratization event, the recipe] / [QLoRA /
// infivelines.com]: gradients flow back through the frozen quantised base
// without updating it; the base is dequantised on the fly.
//
// The reduction here runs over the output features n, while the packed
// weight is stored k-contiguous (row n holds blocks along k).  Each block
// tile decodes a 64 (n) x 256 (k) slab -- one NF4 block per thread, the same
// decode as the forward pass -- and writes it to LDS as it is laid out in
// memory (16-byte stores of 8 consecutive k).  The MFMA operand wants the
// transpose (8 consecutive n of one k per lane), which the LDS transpose
// read ds_read_b64_tr_b16 delivers: within each 16-lane group it hands lane
// i element i % 4 of the 8-byte chunks addressed by lanes i/4, 4 + i/4,
// 8 + i/4 and 12 + i/4, so pointing lane j at row n0 + j/4, column
// k0 + 4 (j % 4) gives lane i the four values of column k0 + i at rows
// n0..n0+3.  dy tiles go to LDS as in the forward pass.
//
// The adapter term uses the same accumulators: with gs = [hi | lo] the bf16
// split of s . dy . B, gs . [A ; A] is run as 2r extra reduction rows.
//
// Block tile 256 (k) x 256 (m), 64 reduction rows per stage; 4 waves in a
// 2 x 2 grid of 128 x 128; two LDS stages of (W slab, dy tile).  (Small-M
// shapes use 256 x 128, or the narrow 128 x 128 tile described at KW.)  As in the
// forward pass, the next slab is decoded while the current one multiplies,
// codes are fetched two slabs ahead, out-of-range rows are clamped rather
// than branched around, and small outputs split the reduction over blocks
// that write fp32 partials.

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int TILE = 256;
constexpr int RT = 64;  // reduction rows per stage
constexpr int ROW_CHUNKS = RT / 8;
// W slab row stride in LDS, bytes: 512 of data plus 64 of pad (144 dwords,
// 16 mod 64 banks), with the 16-byte pieces of row r XOR-swizzled by
// (r / 2) mod 4 within each 64-byte window (slab_swz).  Reads and writes
// see the banks differently (measured with the LDS bank-conflict counter
// on the exact access patterns): a transpose read serves 32 lanes (4 rows
// x 64 contiguous bytes) per cycle across all 64 banks, a 16-byte store
// 8 lanes (8 rows at one column) per cycle across 32 banks, i.e. banks
// taken mod 32.  With the 144-dword stride rows r and r + 2 coincide mod
// 32, so the swizzle has to tell them apart: (r / 2) mod 4 gives the 8
// rows of a store cycle 8 distinct 16-byte bank groups, and the 4 rows of
// a transpose read stay in their own 16-bank quarters.  (The former
// (r / 4) mod 4 swizzle left the stores 2-way conflicted -- half of the dX
// kernel's LDS cycles were conflict cycles; a plain 12-mod-64 stride,
// before that, made the four rows of a transpose read overlap.)
constexpr int WROW = 576;
__device__ __forceinline__ int slab_swz(int row) { return ((row >> 1) & 3) << 4; }

struct DxParams {
  const uint8_t* codes;   // NF4 weight (WF = kWeightNf4 or kWeightNf4Centred)
  const uint8_t* qscale;
  const float* step;
  const float* dq_mean;   // the mean-centred scale format's mean (or null)
  const uint16_t* wbf;    // bf16 weight [N, K] (WF = kWeightBf16)
  const uint8_t* keep;    // LoRA dropout keep bits [M, K / 8] (DROP)
  const uint16_t* dy;
  const uint16_t* gs;
  const uint16_t* A;
  uint16_t* dx;    // bf16 output
  float* part;     // fp32 partials: [splits][M][K] (uniform split) or
                   // [tail_s][tail_q][TM][256] (split tail)
  int64_t M, N, K;
  int r;
  int splits;      // uniform schedule: reduction splits
  int64_t full;    // split-tail schedule: whole tiles
  int tail_q, tail_s;
  Nf4Levels L;
};

__device__ __forceinline__ int64_t clamp_row(int64_t v, int64_t hi) { return v < hi ? v : hi - 1; }

// dy tile: [256 m][64 n], rows 128 B (an even row covers banks 0..31, an
// odd one banks 32..63).  A 16-byte read serves 16 consecutive rows at one
// logical chunk per LDS cycle; xor-swizzling the chunk with (row / 2) mod 8
// gives each pair of rows its own chunk, so those 16 lanes hit all 64 banks.
__device__ __forceinline__ int rk(int row, int chunk) {
  return row * ROW_CHUNKS + (chunk ^ ((row >> 1) & 7));
}

// s_waitcnt immediate: wait until at most `vm` vector-memory and `lgkm` LDS
// operations of this wave are outstanding (expcnt left free).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

}  // namespace

// MS: 32-wide token subtiles per wave; MS = 4 is the 256 (k) x 256 (m)
// tile, MS = 2 the 256 x 128 tile for small-M shapes (twice the output tiles,
// so half the reduction splits and half their fp32 partials).
//
// WF: the weight's format.  kWeightNf4Centred decodes as kWeightNf4 with
// the mean-centred format's block scale.  kWeightBf16 (the unquantised comparison layer)
// loads each thread's 64 bf16 of the slab row instead of decoding a block;
// the values reach the slab at the same points of the schedule.
//
// DROP (LoRA dropout): the adapter term of dX is masked elementwise by the
// keep bits, the base term is not.  Both share the accumulators, so the
// adapter rows run first, the accumulators are masked, and the base
// reduction adds onto them: the sum is still rounded once.
//
// DT: the 16-bit compute type (Bf16T, or F16T for the fp16 variant).
//
// KW: k extent of the block tile.  256 as above; 128 (NF4 only, used with
// MS = 2: a 128 (k) x 128 (m) tile for small-M shapes) gives each thread
// half an NF4 block -- the 32 values of its slab row at k quarter kq -- so
// a thread decodes half as many weights per MFMA; each wave then owns
// 64 (k) x 64 (m).  The slab rows shrink to 256 bytes + 64 of pad, 80
// dwords = 16 mod 64 banks, swizzled like the wide slab.
template <int MS, int WF, bool DROP, class DT, int KW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dx_gemm_kernel(DxParams p) {
  constexpr bool NF4 = WF != kWeightBf16;  // an NF4 weight (either scale format)
  constexpr bool CTR = WF == kWeightNf4Centred;
  constexpr bool HALF = KW == 128;
  static_assert(KW == TILE || (HALF && NF4), "half blocks per thread need the NF4 weight");
  constexpr int NI = KW / 64;         // 32-column (k) MFMA tiles per wave
  constexpr int NCH = KW / 32;        // 8-value chunks each thread decodes
  constexpr int WR = HALF ? 320 : WROW;  // W slab row stride, bytes
  constexpr int WST = RT * WR;           // bytes per W stage
  constexpr int TM = 64 * MS;   // token rows of the block tile
  constexpr int XR = TM / 32;   // dy rows staged per thread
  // one LDS array: two W^T stages, then two dy stages (the epilogue reuses
  // it from the start)
  constexpr int WT_U4 = 2 * WST / 16;
  __shared__ u32x4_t lds[WT_U4 + 2 * TM * ROW_CHUNKS];
  char* const wbase = reinterpret_cast<char*>(&lds[0]);
  u32x4_t(*dyt)[TM * ROW_CHUNKS] = reinterpret_cast<u32x4_t(*)[TM * ROW_CHUNKS]>(&lds[WT_U4]);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: scalar addressing
  const int lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int wk = wave & 1, wm = wave >> 1;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m_tiles = (M + TM - 1) / TM, k_tiles = (K + KW - 1) / KW;
  const BlockWork bw = block_work(blockIdx.x, (int64_t)gridDim.x, m_tiles, k_tiles, p.splits,
                                  p.full, p.tail_q, p.tail_s);
  const int64_t k0 = bw.n * KW;
  const int64_t m0 = bw.m * TM;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const ScaleFmt fmt = scale_fmt(CTR ? p.dq_mean : nullptr);
  // the merge selector's byte indices 0..3 in a register: the selector is
  // then one v_and_or_b32 (a form that cannot carry two literal constants)
  // instead of an and and an or
  uint32_t kidx;
  asm volatile("v_mov_b32 %0, 0x03020100" : "=v"(kidx));

  f32x16_t acc[NI][MS];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MS; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int z = bw.z, nz = bw.nz;
  const int64_t nst = N / RT;
  const int64_t st0 = nst * z / nz, st1 = nst * (z + 1) / nz;

  // this thread decodes reduction row 16 wave + lane % 16 of the slab, k
  // quarter lane / 16 (so the 16 lanes of one LDS store cycle write 16
  // rows); a quarter past K is clamped to the last in-range quarter (never
  // stored)
  const int wr = 16 * wave + (lane & 15);
  const int kq = lane >> 4;
  const int64_t kcol_raw = k0 + (KW / 4) * kq;
  const bool kcol_ok = kcol_raw < K;
  const int64_t kcol = kcol_ok ? kcol_raw : K - KW / 4;
  // dy rows m0 + (t >> 3) + 32 j through a buffer descriptor: rows past M
  // read as zero
  const __amdgpu_buffer_rsrc_t yres = make_rsrc(p.dy, (uint32_t)(M * N * 2));
  // The dy tile reaches LDS by DMA (buffer loads that write LDS directly):
  // instruction q of wave w fills tile rows 8 (XR w + q) .. + 7 of a stage,
  // lane i its 16 bytes at 16 i -- row 8 (XR w + q) + i / 8 at physical
  // chunk i % 8, which holds logical chunk (i % 8) ^ ((row / 2) % 8), the
  // swizzled layout of rk -- so each lane fetches that chunk.  The row is
  // in the lane offset (rows past M lie beyond the descriptor and read as
  // zero), the slab's column in the scalar offset.
  // (a fixed-size array: a lambda capturing one whose size depends on the
  // template arguments, used as a buffer-load operand, fails to substitute
  // in the host pass, which then silently drops the kernel's host stub)
  static_assert(XR <= 8, "dy DMA offsets");
  uint32_t yvoff[8];
#pragma unroll
  for (int q = 0; q < XR; ++q) {
    const int row = 8 * (XR * wave + q) + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    yvoff[q] = (uint32_t)(((m0 + row) * N + 8 * lc) * 2);
  }
  // NF4 codes and scale bytes likewise: the lane's element offset within a
  // slab is fixed, the slab's first element is uniform
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(p.codes, (uint32_t)((N * K) >> 1));
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(p.qscale, (uint32_t)((N * K) >> 6));
  const int64_t lidx = (int64_t)wr * K + kcol;
  const uint32_t cvoff = (uint32_t)(lidx >> 1), qvoff = (uint32_t)(lidx >> 6);

  // The scale byte and its step stay raw until the tile is decoded (an
  // iteration later): forming s' here would make the wave wait for this
  // prefetch -- and, since loads return in order, for every load before it.
  struct CodesNf4 {
    u32x4_t c0, c1;
    uint32_t q;
    float st;
  };
  struct CodesHalf {
    u32x4_t c0;  // the codes of the thread's 32 values
    uint32_t q;
    float st;
  };
  struct WordsBf16 {
    u32x4_t w[8];  // chunk c: the 8 values at k = kcol + 8c .. + 7
  };
  using Codes =
      std::conditional_t<NF4, std::conditional_t<HALF, CodesHalf, CodesNf4>, WordsBf16>;
  // code word of chunk ch (8 values) of the thread's codes
  auto word = [](const Codes& c, int ch) -> uint32_t {
    if constexpr (HALF)
      return c.c0[ch & 3];
    else if constexpr (NF4)
      return (ch < 4 ? c.c0 : c.c1)[ch & 3];
    else
      return 0u;
  };
  auto load_codes = [&](int64_t st, Codes& c) {
    // first element of the thread's values (a whole block, or half of one):
    // slab base sb (a multiple of 64 K) + the lane's lidx
    const int64_t sb = st * RT * K;
    if constexpr (NF4) {
      c.c0 = buffer_load16(cres, cvoff, (uint32_t)(sb >> 1));
      if constexpr (!HALF) c.c1 = buffer_load16(cres, cvoff + 16u, (uint32_t)(sb >> 1));
      c.q = buffer_load1(qres, qvoff, (uint32_t)(sb >> 6));
      c.st = p.step[(sb + lidx) >> 14];
    } else {
      const int64_t idx = sb + lidx;
      const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(p.wbf + idx);
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = wp[i];
    }
  };
  auto dma_dy = [&](u32x4_t* stage, int64_t st) {
#pragma unroll
    for (int q = 0; q < XR; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          yres, (__attribute__((address_space(3))) void*)(stage + 8 * (XR * wave + q) * ROW_CHUNKS),
          16, yvoff[q], (uint32_t)(st * RT * 2), 0, 0);
  };
  // vector-memory operations of one load_codes (the DMA waits below count
  // only the codes issued after a dy DMA)
  constexpr int kCodeOps = NF4 ? (HALF ? 3 : 4) : 8;
  // store 8 consecutive-k 16-bit values (chunk c of this thread's NCH) of
  // reduction row `wr` into the W slab
  // (stage given as its base: the main loop passes restrict-qualified
  // stage pointers, which tell the compiler the dy DMA's destination is
  // disjoint from everything an iteration reads, so it places no wait for
  // the DMA before those reads)
  auto store8p = [&](char* stage_base, int c, const u32x4_t v) {
    *reinterpret_cast<u32x4_t*>(stage_base + wr * WR +
                                ((((KW / 4) * kq + 8 * c) * 2) ^ slab_swz(wr))) = v;
  };
  auto store8 = [&](int stage, int c, const u32x4_t v) { store8p(wbase + stage * WST, c, v); };
  // A operand of MFMA step kk, k sub-tile i: lane l holds column
  // (KW / 2) wk + 32 i + l % 32 at reduction rows 16 kk + 8 (l / 32) + 0..7, from
  // two transpose reads (rows +0..3 and +4..7).  As provider, lane j of
  // 16-lane group g points at row 8 (g / 2) + j / 4 (+ 4 for the second
  // read), column 16 (g % 2) + 4 (j % 4).
  // (The swizzle term of a row does not change with kk, as 16 kk is a
  // multiple of 8 rows, nor with i, which moves by whole 64-byte windows.)
  const int tg = lane >> 4, tj = lane & 15;
  const int a_row = 8 * (tg >> 1) + (tj >> 2);
  const int a_col = ((KW / 2) * wk + 16 * (tg & 1) + 4 * (tj & 3)) * 2;
  const int a_off0 = a_row * WR + (a_col ^ slab_swz(a_row));
  const int a_off1 = (a_row + 4) * WR + (a_col ^ slab_swz(a_row + 4));
  auto read_ap = [&](const char* stage_base, int kk, int i) -> u32x4_t {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const int o = 16 * kk * WR + 64 * i;
    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(stage_base + o + a_off0));
    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(stage_base + o + a_off1));
    const u32x2_t h0 = __builtin_bit_cast(u32x2_t, r0), h1 = __builtin_bit_cast(u32x2_t, r1);
    const u32x4_t v = {h0[0], h0[1], h1[0], h1[1]};
    return v;
  };
  auto read_a = [&](int stage, int kk, int i) { return read_ap(wbase + stage * WST, kk, i); };
  auto mfma_step = [&](int stage, int kk) {
    const int ch = 2 * kk + lg;
    u32x4_t a[NI], b[MS];
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = read_a(stage, kk, i);
#pragma unroll
    for (int j = 0; j < MS; ++j) b[j] = dyt[stage][rk(32 * MS * wm + 32 * j + lr, ch)];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < MS; ++j) acc[i][j] = DT::mfma32(a[i], b[j], acc[i][j]);
  };

  // --- adapter rows: gs [M, 2r] against [A ; A] (last split only) ---
  const int r = p.r;
  auto adapter_rows = [&]() {
    const int ext_tiles = (2 * r + RT - 1) / RT;
    const int64_t m = clamp_row(m0 + (t % TM), M);
    for (int e = 0; e < ext_tiles; ++e) {
      // W^T side: reduction row c = e*64 + wr is A's row (c mod r), zero past 2r
      const int c = e * RT + wr;
      const bool row_ok = c < 2 * r;
      const int arow = c < r ? c : c - r;
#pragma unroll
      for (int q = 0; q < NCH; ++q)
        store8(0, q, row_ok ? *reinterpret_cast<const u32x4_t*>(p.A + (int64_t)arow * K + kcol + 8 * q)
                              : zero);
      // dy side: rows m, columns c of gs
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int col = e * RT + 8 * q;
        if (t < TM)
          dyt[0][rk(t, q)] =
              col < 2 * r ? *reinterpret_cast<const u32x4_t*>(p.gs + m * 2 * r + col) : zero;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) mfma_step(0, kk);
      __syncthreads();
    }
  };

  // Dropout mask on the accumulators: lane (lr, lg) of acc[i][j] holds
  // token m0 + 32 MS wm + 32 j + lr and, in register v, column
  // k0 + (KW / 2) wk + 32 i + 8 (v / 4) + 4 lg + v % 4 -- 16 bits of the
  // 32-bit keep word of that token row at column k0 + (KW / 2) wk + 32 i.
  // Rows past M read zero (not stored); columns past K are not stored.
  auto mask_acc = [&]() {
    const __amdgpu_buffer_rsrc_t kres = make_rsrc(p.keep, (uint32_t)(M * K / 8));
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < MS; ++j) {
        const int64_t m = m0 + 32 * MS * wm + 32 * j + lr;
        const int64_t kw = k0 + (KW / 2) * wk + 32 * i;
        // the lane half's bits first, so every bit index below is a constant
        const uint32_t word = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                  kres, (int)(uint32_t)(m * (K / 8) + kw / 8), 0, 0) >>
                              (4 * lg);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int bit = 8 * (v >> 2) + (v & 3);
          acc[i][j][v] = ((word >> bit) & 1u) ? acc[i][j][v] : 0.0f;
        }
      }
  };
  if constexpr (DROP) {
    if (z == nz - 1) {
      adapter_rows();
      mask_acc();
    }
  }

  if (st0 < st1) {
    // Register sets indexed by slab parity (relative to st0), loaded at the
    // top of the iteration two slabs ahead into the set that was just
    // consumed; the loop is unrolled by two so the parity is a constant and
    // no register holding an in-flight load is copied.
    const int64_t last = st1 - 1;
    auto cl = [&](int64_t v) { return v < last ? v : last; };
    Codes C[2];
    dma_dy(dyt[0], st0);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(st0, C[0]);
    if constexpr (NF4) {
      const Nf4Lut lut = nf4_make_lut<DT>(p.L, (CTR ? nf4_block_scale(C[0].q, C[0].st, fmt) : nf4_block_scale(C[0].q, C[0].st)));
#pragma unroll
      for (int c = 0; c < NCH; ++c) store8(0, c, nf4_decode8(lut, word(C[0], c)));
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) store8(0, c, C[0].w[c]);
    }
    load_codes(cl(st0 + 1), C[1]);
    // slab st0's dy DMA (older than these codes) has landed
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kCodeOps, 0));
    __syncthreads();

    // Hand-scheduled iteration, as in the forward pass: each of the MFMAs
    // of the slab is followed by a fixed share of the 64 units of other
    // work and a scheduling fence -- the table of slab st+1's block (units
    // 0..7) and the decode of its NCH code words (6 units each, about 5
    // vector ops per unit; the last one stores the 8 values into the W
    // slab) -- and the operand reads of step kk+1 ride in the last slots of
    // step kk, so the vector work fits in the MFMAs' shadow.  Slab st+1's
    // dy tile is DMA'd into the other stage at the top (that stage was last
    // read in the previous iteration, before its closing barrier) and
    // waited for before this iteration's closing barrier; the codes go two
    // slabs ahead into registers.
    auto iteration = [&](int64_t st, auto parity, const u32x4_t* __restrict__ y_rd,
                         u32x4_t* __restrict__ y_fill, const char* __restrict__ w_rd,
                         char* __restrict__ w_fill) {
      constexpr int cur = decltype(parity)::value, nxt = cur ^ 1;
      dma_dy(y_fill, cl(st + 1));
      __builtin_amdgcn_sched_barrier(0);
      load_codes(cl(st + 2), C[cur]);
      const Codes& cn = C[nxt];
      constexpr int SPK = NI * MS;  // MFMAs (slots) per k step
      constexpr int NRD = NI + MS;  // operand reads per k step
      constexpr int DEC = 8 + 6 * NCH;  // table and decode units
      static_assert(SPK >= NRD && DEC <= 64, "unit schedule");
      u32x4_t op[2][2][4];          // [buffer][a|b][i]
      auto read_op = [&](int kk, int buf, int q) {
        const int ch = 2 * kk + lg;
        if (q < NI)
          op[buf][0][q] = read_ap(w_rd, kk, q);
        else
          op[buf][1][q - NI] = y_rd[rk(32 * MS * wm + 32 * (q - NI) + lr, ch)];
      };
#pragma unroll
      for (int q = 0; q < NRD; ++q) read_op(0, 0, q);

      uint32_t pk[8];
      Nf4Lut lut;
      float sc = 0.0f;
      uint32_t dn0 = 0, dn1 = 0, nh = 0, pick = 0, la = 0, lb = 0;
      u32x4_t dv = zero;
      auto lookup_a = [&](uint32_t n) {  // low-byte planes of 4 codes
        nh = n & 0x07070707u;
        pick = ((n >> 1) & 0x04040404u) | kidx;
        la = perm(lut.lo[1], lut.lo[0], nh);
        lb = perm(lut.lo[3], lut.lo[2], nh);
      };
      auto lookup_b = [&](uint32_t n, uint32_t& o01, uint32_t& o23) {  // high bytes, merge
        const uint32_t lo = perm(lb, la, pick);
        const uint32_t hi =
            perm(perm(lut.hi[3], lut.hi[2], nh), perm(lut.hi[1], lut.hi[0], nh), pick);
        o01 = perm(hi, lo, 0x05010400u);
        o23 = perm(hi, lo, 0x07030602u);
      };
      auto unit = [&](int u) {
        if constexpr (!NF4) {
          // no table or decode: a chunk's store sits where its decode ends
          if (u >= 8 && u < DEC) {
            if ((u - 8) % 6 == 5) store8p(w_fill, (u - 8) / 6, cn.w[(u - 8) / 6]);
          }
        } else if (u < 4) {
          if (u == 0) sc = CTR ? nf4_block_scale(cn.q, cn.st, fmt) : nf4_block_scale(cn.q, cn.st);
          pk[2 * u] = DT::pack2(p.L.v[4 * u] * sc, p.L.v[4 * u + 1] * sc);
          pk[2 * u + 1] = DT::pack2(p.L.v[4 * u + 2] * sc, p.L.v[4 * u + 3] * sc);
        } else if (u < 8) {
          const int j = u - 4;
          lut.lo[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
          lut.hi[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
        } else if (u < DEC) {
          const int c = (u - 8) / 6, w = (u - 8) % 6;
          const uint32_t v = word(cn, c);
          switch (w) {
            case 0: {
              // codes 0..3 (dn0) and 4..7 (dn1) of the word, one per byte in
              // the low nibble; the high nibbles carry the neighbouring code,
              // which no lookup reads (they use bits 0..2, the merge bit 3)
              const uint32_t od = v >> 4;
              dn0 = perm(od, v, 0x05010400u);
              dn1 = perm(od, v, 0x07030602u);
              break;
            }
            case 1: lookup_a(dn0); break;
            case 2: { uint32_t o0, o1; lookup_b(dn0, o0, o1); dv[0] = o0; dv[1] = o1; break; }
            case 3: lookup_a(dn1); break;
            case 4: { uint32_t o2, o3; lookup_b(dn1, o2, o3); dv[2] = o2; dv[3] = o3; break; }
            default: store8p(w_fill, c, dv); break;
          }
        }
      };
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int s2 = 0; s2 < SPK; ++s2) {
          const int i = s2 / MS, j = s2 % MS;
          acc[i][j] = DT::mfma32(op[kk & 1][0][i], op[kk & 1][1][j], acc[i][j]);
          if (kk < 3 && s2 >= SPK - NRD) read_op(kk + 1, (kk + 1) & 1, s2 - (SPK - NRD));
          constexpr int UPS = 16 / SPK;  // units per slot: 64 units over 4 SPK slots
#pragma unroll
          for (int e = 0; e < UPS; ++e) unit(UPS * (SPK * kk + s2) + e);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // slab st+1's dy DMA has landed (only this iteration's codes, issued
      // after it, may still be in flight)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(kCodeOps, 0));
      __syncthreads();
    };
    u32x4_t* const Y0 = dyt[0];
    u32x4_t* const Y1 = dyt[1];
    char* const W0 = wbase;
    char* const W1 = wbase + WST;
    for (int64_t st = st0; st < st1; st += 2) {
      iteration(st, std::integral_constant<int, 0>(), Y0, Y1, W0, W1);
      if (st + 1 < st1) iteration(st + 1, std::integral_constant<int, 1>(), Y1, Y0, W1, W0);
    }
  }

  if constexpr (!DROP) {
    if (z == nz - 1) adapter_rows();
  }

  // --- epilogue: D[k][m] -> dx[m][k] (or the split's fp32 partial) ---
  __syncthreads();  // the LDS stages are free from here on
  float* scratch = reinterpret_cast<float*>(&lds[0]) + wave * epi_floats<NI>();
  if (bw.tail >= 0)  // tile-local [TM][KW] partial
    store_acc_tile<NI, MS, DT>(acc, scratch, (KW / 2) * wk, 32 * MS * wm, K - k0, M - m0, true,
                               p.part + ((int64_t)z * p.tail_q + bw.tail) * TM * KW, nullptr,
                               KW, lane);
  else
    store_acc_tile<NI, MS, DT>(acc, scratch, k0 + (KW / 2) * wk, m0 + 32 * MS * wm, K, M,
                               nz > 1, nz > 1 ? p.part + (int64_t)z * M * K : nullptr, p.dx, K,
                               lane);
}

// block tile (k x tokens), dropout mask or not, compute type for a weight
// format: fp16 with the NF4 weight and no mask only, the narrow tile with
// the NF4 weight only
template <int WF>
static void launch_dx_kernel(const GemmConfig& cfg, bool f16, bool drop, dim3 grid,
                             hipStream_t s, const DxParams& p) {
  constexpr bool Q = WF != kWeightBf16;
  auto go = [&](auto ms, auto kw) {
    constexpr int MS = decltype(ms)::value, KW = decltype(kw)::value;
    if constexpr (Q) {
      if (f16) {
        hipLaunchKernelGGL((dx_gemm_kernel<MS, WF, false, F16T, KW>), grid, dim3(256), 0, s, p);
        return;
      }
    }
    if (drop)
      hipLaunchKernelGGL((dx_gemm_kernel<MS, WF, true, Bf16T, KW>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((dx_gemm_kernel<MS, WF, false, Bf16T, KW>), grid, dim3(256), 0, s, p);
  };
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (cfg.tn != TILE) {
    if constexpr (Q) go(I2(), std::integral_constant<int, 128>());
  } else if (cfg.tm == 256) {
    go(I4(), std::integral_constant<int, TILE>());
  } else {
    go(I2(), std::integral_constant<int, TILE>());
  }
}

hipError_t launch_dx_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const float* dq_mean, const uint16_t* wbf, const uint8_t* keep,
                          const uint16_t* dy,
                          const uint16_t* gs, const uint16_t* A, uint16_t* dx, float* part,
                          int64_t M, int64_t N, int64_t K, int r, const Nf4Levels& L,
                          hipStream_t s, bool f16) {
  // output M x K, reduction N: the forward GEMM's schedule with the roles
  // of N and K exchanged
  const bool nf4 = wbf == nullptr, drop = keep != nullptr && r > 0;
  const GemmConfig cfg = gemm_config(M, K, N, nf4);
  if (gemm_partial_bytes(cfg, M, K) > 0 && part == nullptr) return hipErrorInvalidValue;
  DxParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.dq_mean = dq_mean;
  p.wbf = wbf;
  p.keep = keep;
  p.dy = dy;
  p.gs = gs;
  p.A = A;
  p.dx = dx;
  p.part = part;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  p.splits = cfg.splits;
  p.full = cfg.full;
  p.tail_q = cfg.tail_q;
  p.tail_s = cfg.tail_s;
  p.L = L;
  const int64_t blocks = gemm_blocks(cfg, M, K);
  const dim3 grid((unsigned)blocks);
  if (!nf4)
    launch_dx_kernel<kWeightBf16>(cfg, false, drop, grid, s, p);
  else if (dq_mean)
    launch_dx_kernel<kWeightNf4Centred>(cfg, f16, drop, grid, s, p);
  else
    launch_dx_kernel<kWeightNf4>(cfg, f16, drop, grid, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_reduce(cfg, part, M, K, dx, s, f16);
}

}  // namespace qlora
