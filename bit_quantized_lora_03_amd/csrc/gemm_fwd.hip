// Fused forward GEMM: y = x . deq(W)^T + (alpha/r) . (x . A^T) . B^T (gfx950).
//
// [QLoRA / infivelines.com]: the 4-bit base is dequantised to bf16 one block
// at a time inside the matrix multiply, and the adapters stay in full
// precision.  One 64-wide k tile of a weight row is exactly one NF4 block,
// so each thread decodes one weight row's block per k tile with that block's
// own 16-entry table, and the decoded values go straight into the MFMA
// operand registers: the weight never passes through LDS.  Only the
// activation tile, which all four waves share, is staged in LDS.
//
// The adapter term rides on the same accumulators: with xs = [hi | lo] the
// bf16 split of s . x . A^T (hi + lo equals the fp32 value to 2^-17), the
// product xs . [B | B]^T runs as 2r extra reduction columns after the base
// reduction, so y is rounded to bf16 exactly once.
//
// Block tile 256 (n) x TM (m) x 64 (k), TM = 256 or 128; 4 waves, wave w
// owning weight rows 64 w .. 64 w + 63 against all TM tokens (2 x TM/32
// MFMA 32x32x16 tiles, fp32 accumulate, one wave per SIMD); small-M
// shapes may use a narrow 128 (n) x 128 (m) tile instead (RW below).
// Thread t decodes row 64 w + t of its wave into eight 8-value chunks.
// MFMA step kk of a k tile takes, in lanes 0..31, k chunk kk and, in
// lanes 32..63, chunk 4 + kk (the reduction order inside a tile is free, as
// long as both operands use the same one), so lane l needs chunk kk of row
// l % 32 and lane l + 32 chunk 4 + kk of it: one v_permlane32_swap per
// register pair exchanges the halves decoded by the other 32 lanes.
//
// Pipeline: the activation tile goes through a 4-stage LDS ring, filled by
// DMA three k tiles ahead, so one barrier per k tile covers both hazards
// and the B operands of the next tile's first step can be read before that
// barrier.  While the MFMAs of tile t run, the same waves decode tile t+1's
// codes (loaded four tiles ahead) in small, fixed pieces placed between the
// MFMAs, so the matrix cores and the vector ALUs work at the same time.
// Out-of-range rows are clamped to the last valid row instead of branched
// around, so the loop body is a single basic block; their results are
// never stored.
//
// When the output has too few tiles to fill the chip, the k range is split
// over blocks that write fp32 partials; splitk_reduce adds them in a fixed
// order and rounds once.

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int TILE_N = 256;  // n extent of a block tile
constexpr int KT = 64;       // k extent of one tile (= one NF4 block)
constexpr int ROW_CHUNKS = KT / 8;  // 16-byte chunks per tile row
constexpr int NSTAGE = 4;           // activation ring depth

struct FwdParams {
  const uint8_t* codes;   // NF4 weight (WF = kWeightNf4 or kWeightNf4Centred)
  const uint8_t* qscale;
  const float* step;
  const float* dq_mean;   // the mean-centred scale format's mean (or null)
  const uint16_t* wbf;    // bf16 weight [N, K] (WF = kWeightBf16)
  const uint16_t* x;
  const uint16_t* xs;
  const uint16_t* B;
  uint16_t* y;     // bf16 output
  float* part;     // fp32 partials: [splits][M][N] (uniform split) or
                   // [tail_s][tail_q][TM][256] (split tail)
  int64_t M, N, K;
  int r;
  int splits;      // uniform schedule: reduction splits
  int64_t full;    // split-tail schedule: whole tiles
  int tail_q, tail_s;
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

// s_waitcnt immediate: wait until at most `vm` vector-memory and `lgkm` LDS
// operations of this wave are outstanding (expcnt left free).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// Register v of a and b becomes (lanes 0..31 of a, lanes 0..31 of b) and
// (lanes 32..63 of a, lanes 32..63 of b).
__device__ __forceinline__ void swap_halves(u32x4_t& a, u32x4_t& b, int v) {
  const auto r = __builtin_amdgcn_permlane32_swap(a[v], b[v], false, false);
  a[v] = r[0];
  b[v] = r[1];
}

}  // namespace

// JT: 32-token MFMA tiles per wave; the block tile is 256 (n) x 32 JT (m).
// JT = 8 amortises each decoded weight over 256 tokens; JT = 4 doubles the
// number of output tiles for small-M shapes and so halves the k splits
// (and their fp32 partials) needed to fill the chip.
// WF: the weight's format.  kWeightNf4 decodes each thread's block as
// described above (kWeightNf4Centred likewise, with the mean-centred
// format's block scale); kWeightBf16 (the unquantised comparison layer) loads the
// 64 bf16 of the same row tile instead and skips the table and decode, so
// the two share every other part of the kernel.
// DT: the 16-bit compute type (Bf16T, or F16T for the fp16 variant).
//
// RW: weight rows per wave.  64 (the block tile is 256 n x TM): each lane
// decodes a whole row and the lane halves swap chunks, as described above.
// 32 (the block tile is 128 n x TM, NF4 only; used with TM = 128): lanes l
// and l + 32 share row l % 32 and each decodes just the four chunks its own
// MFMA operand takes (chunks 4 (l / 32) + kk), so a lane decodes half as
// many weights per MFMA and nothing is swapped.  The 128 x 128 tile thus
// has the decode-to-MFMA ratio of the 256 x 256 one while giving small-M
// shapes four times the output tiles (fewer k splits, fewer partials).
template <int JT, int WF, class DT, int RW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(FwdParams p) {
  constexpr bool NF4 = WF != kWeightBf16;  // an NF4 weight (either scale format)
  constexpr bool CTR = WF == kWeightNf4Centred;
  constexpr bool HALF = RW == 32;
  static_assert(RW == 64 || (HALF && NF4), "half rows per lane need the NF4 weight");
  constexpr int NI = RW / 32;   // 32-row MFMA tiles per wave
  constexpr int TN = 4 * RW;    // n extent of the block tile
  // weight ring depth (tiles loaded ahead) and vector loads per weight tile:
  // a bf16 tile is 8 x 16 bytes per thread, so the 256-token tile (whose
  // accumulators leave the fewest registers) keeps two tiles, not four
  constexpr int WD = NF4 ? 4 : (JT == 8 ? 2 : 4);
  constexpr int LC = NF4 ? (HALF ? 3 : 4) : 8;
  constexpr int TM = 32 * JT;             // token rows of the block tile
  constexpr int XR = TM / 32;             // x chunks staged per thread per tile
  constexpr int XST = TM * ROW_CHUNKS;    // u32x4 per ring stage
  constexpr int EPI = 4 * epi_floats<NI>() / 4;  // epilogue scratch, u32x4
  constexpr int LDS_U4 = NSTAGE * XST > EPI ? NSTAGE * XST : EPI;
  __shared__ u32x4_t lds[LDS_U4];
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: scalar addressing
  const int lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m_tiles = (M + TM - 1) / TM, n_tiles = (N + TN - 1) / TN;
  const BlockWork bw = block_work(blockIdx.x, (int64_t)gridDim.x, m_tiles, n_tiles, p.splits,
                                  p.full, p.tail_q, p.tail_s);
  const int64_t n0 = bw.n * TN;
  const int64_t m0 = bw.m * TM;
  const int z = bw.z, nz = bw.nz;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto Xs = [&](int stage, int row, int chunk) -> u32x4_t& {
    return lds[stage * XST + rk(row, chunk)];
  };
  // B operand of MFMA step kk, token tile j: chunk kk (lanes 0..31) or
  // 4 + kk (lanes 32..63) of token 32 j + l % 32
  auto read_b = [&](int stage, int kk, int j) -> u32x4_t {
    return Xs(stage, 32 * j + lr, 4 * lg + kk);
  };

  const ScaleFmt fmt = scale_fmt(CTR ? p.dq_mean : nullptr);
  // k tiles of this split
  const int64_t nkt = K / KT;
  const int64_t kt0 = nkt * z / nz, kt1 = nkt * (z + 1) / nz;

  f32x16_t acc[NI][JT];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < JT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // this thread decodes weight row n0 + t (clamped), or with half rows the
  // half lg of row n0 + 32 wave + lr
  const int64_t wrow = clamp_row(HALF ? n0 + 32 * wave + lr : n0 + t, N);
  const uint16_t* wvals = NF4 ? nullptr : p.wbf + wrow * K;
  const int64_t wblk0 = (wrow * K) >> 6;
  // codes and scale bytes through buffer descriptors: the row's offset is
  // the lane's (fixed), the k tile's the uniform scalar offset
  const __amdgpu_buffer_rsrc_t cres = make_rsrc(p.codes, (uint32_t)((N * K) >> 1));
  const __amdgpu_buffer_rsrc_t qres = make_rsrc(p.qscale, (uint32_t)((N * K) >> 6));
  const uint32_t cvoff = (uint32_t)((wrow * K) >> 1) + (HALF ? 16u * (uint32_t)lg : 0u);
  const uint32_t qvoff = (uint32_t)wblk0;

  // The x tile reaches LDS by DMA (buffer loads that write LDS directly):
  // instruction q of wave w fills the 1 KiB region R = XR w + q of a stage,
  // lane i its 16 bytes at 16 i, i.e. tile row 8 R + i / 8 at physical
  // chunk i % 8, which holds logical chunk (i % 8) ^ ((row / 2) % 8) -- the
  // swizzled layout -- so each lane fetches that chunk.  The swizzle term
  // is (4 (R % 2) + i / 16) % 8, so lanes need one offset for even and one
  // for odd R.  Rows past M lie beyond the descriptor and read as zero.
  // The bounds check covers the per-lane offset only (not the scalar one),
  // so every row term goes into the lane offset and the scalar offset
  // carries the k position alone.
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(p.x, (uint32_t)(M * K * 2));
  uint32_t xvoff[2];
#pragma unroll
  for (int odd = 0; odd < 2; ++odd) {
    const int c = (lane & 7) ^ ((4 * odd + (lane >> 4)) & 7);
    xvoff[odd] = (uint32_t)((m0 + 8 * XR * wave + (lane >> 3)) * K * 2 + 16 * c);
  }
  auto dma_x = [&](u32x4_t* stage, int64_t kt, int q) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xres, (__attribute__((address_space(3))) void*)(stage + 64 * (XR * wave + q)), 16,
        xvoff[q & 1] + (uint32_t)(q * 8 * K * 2), (uint32_t)(kt * KT * 2), 0, 0);
  };

  // The scale byte and its step stay raw until the tile is decoded:
  // forming s' at load time would make the wave wait for this prefetch --
  // and, since loads return in order, for every load before it.
  struct CodesNf4 {
    u32x4_t c0, c1;
    uint32_t q;
    float st;
  };
  struct CodesHalf {
    u32x4_t c;  // word i: the codes of chunk 4 lg + i of the tile
    uint32_t q;
    float st;
  };
  struct WordsBf16 {
    u32x4_t w[8];  // chunk c: the 8 values at k = 8c .. 8c + 7 of the tile
  };
  using Codes =
      std::conditional_t<NF4, std::conditional_t<HALF, CodesHalf, CodesNf4>, WordsBf16>;
  auto load_codes = [&](int64_t kt, Codes& c) {
    if constexpr (HALF) {
      c.c = buffer_load16(cres, cvoff, (uint32_t)(kt * (KT / 2)));
      c.q = buffer_load1(qres, qvoff, (uint32_t)kt);
      c.st = p.step[(wblk0 + kt) >> 8];
    } else if constexpr (NF4) {
      c.c0 = buffer_load16(cres, cvoff, (uint32_t)(kt * (KT / 2)));
      c.c1 = buffer_load16(cres, cvoff + 16u, (uint32_t)(kt * (KT / 2)));
      c.q = buffer_load1(qres, qvoff, (uint32_t)kt);
      c.st = p.step[(wblk0 + kt) >> 8];
    } else {
      const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(wvals + kt * KT);
#pragma unroll
      for (int i = 0; i < 8; ++i) c.w[i] = wp[i];
    }
  };
  auto store_x = [&](int stage, int q, const u32x4_t& v) {
    Xs(stage, (t >> 3) + 32 * q, t & 7) = v;
  };

  if (kt0 < kt1) {
    // Rings indexed by tile number mod 4 (relative to kt0): LDS stage q
    // and code set C[q] belong to a tile with that residue.  x tiles are
    // DMA'd three tiles ahead and codes loaded at the end of the iteration
    // four tiles earlier.  Vector loads complete in order, so a wait for
    // any load is also a wait for every older one; the order (x chunks,
    // then codes) and the one wait per iteration are arranged so that x
    // gets one to two iterations and codes (whose first touch of a weight
    // line comes from HBM) two.  The loop is unrolled by four so every ring index is a
    // constant and no register holding an in-flight load is ever copied (a
    // copy would make the compiler wait for the load).  Prefetch indices
    // are clamped into the split, so loads are unconditional.
    const int64_t last = kt1 - 1;
    auto cl = [&](int64_t v) { return v < last ? v : last; };
    Codes C[WD];
    u32x4_t Ap[2][NI];   // A operands of a step: [step parity][i]
    u32x4_t op[2][JT];   // B operands, by step parity

    // Decode state.  The weights are decoded just in time: during step kk
    // the waves decode the chunk pair step kk+1 needs (pair 0 of the next
    // tile, after that tile's table, during step 3), so only two steps of A
    // operands are ever held.
    uint32_t pk[8];
    Nf4Lut lut;
    float sc = 0.0f;
    uint32_t dn0 = 0, dn1 = 0, nh = 0, pick = 0, la = 0, lb = 0;
    u32x4_t dlo = zero, dhi = zero;
    // the merge selector's byte indices 0..3, held in a register so that the
    // selector takes one v_and_or_b32 (a vector-ALU form that cannot carry
    // two literal constants) instead of an and and an or
    uint32_t kidx;
    asm volatile("v_mov_b32 %0, 0x03020100" : "=v"(kidx));
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
    auto decode_part = [&](uint32_t v, int w, u32x4_t& d) {
      switch (w) {
        case 0: {
          // codes 0..3 (dn0) and 4..7 (dn1) of the word, one per byte in the
          // low nibble; the high nibbles carry the neighbouring code, which
          // no lookup reads (they use bits 0..2, the merge bit 3)
          const uint32_t od = v >> 4;
          dn0 = perm(od, v, 0x05010400u);
          dn1 = perm(od, v, 0x07030602u);
          break;
        }
        case 1: lookup_a(dn0); break;
        case 2: { uint32_t o0, o1; lookup_b(dn0, o0, o1); d[0] = o0; d[1] = o1; break; }
        case 3: lookup_a(dn1); break;
        default: { uint32_t o2, o3; lookup_b(dn1, o2, o3); d[2] = o2; d[3] = o3; break; }
      }
    };
    // table unit u (0..7) of a block: four products-and-packs, four perms
    auto table_unit = [&](const Codes& c, int u) {
      if constexpr (!NF4) return;
      else if (u < 4) {
        if (u == 0) sc = CTR ? nf4_block_scale(c.q, c.st, fmt) : nf4_block_scale(c.q, c.st);
        pk[2 * u] = DT::pack2(p.L.v[4 * u] * sc, p.L.v[4 * u + 1] * sc);
        pk[2 * u + 1] = DT::pack2(p.L.v[4 * u + 2] * sc, p.L.v[4 * u + 3] * sc);
      } else {
        const int j = u - 4;
        lut.lo[j] = perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
        lut.hi[j] = perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
      }
    };
    // pair unit w (0..11) of chunk pair pr: the decode of code words pr and
    // 4 + pr (5 units each, about 5 vector ops per unit), then the
    // lane-half exchange (2 units) that makes them step pr's A operands
    auto pair_unit = [&](const Codes& c, int pr, int w, u32x4_t (&dst)[NI]) {
      if constexpr (HALF) {
        // word pr of the lane's own codes is its operand for step pr
        if (w < 5) decode_part(c.c[pr], w, dlo);
        if (w == 4) dst[0] = dlo;
      } else {
        if constexpr (!NF4) {
          if (w == 0) {
            dlo = c.w[pr];
            dhi = c.w[4 + pr];
          }
        }
        if (w < 5) {
          if constexpr (NF4) decode_part(c.c0[pr], w, dlo);
        } else if (w < 10) {
          if constexpr (NF4) decode_part(c.c1[pr], w - 5, dhi);
        } else {
          const int v = 2 * (w - 10);
          swap_halves(dlo, dhi, v);
          swap_halves(dlo, dhi, v + 1);
          if (w == 11) {
            dst[0] = dlo;
            dst[NI - 1] = dhi;
          }
        }
      }
    };
    constexpr int NUP = HALF ? 5 : 12;  // units of one pair (one word with half rows)

    // Prologue: codes of tiles kt0..kt0+3, x tiles kt0..kt0+2, the table
    // and first pair of tile kt0; then wait for x tiles kt0 and kt0+1.  The
    // issue order (kept by scheduling fences) ends like an iteration's: x
    // tile kt0+2, then the codes of kt0+3, which the waits below count on.
    // (With a weight ring of depth WD the middle loads are tiles
    // kt0+1 .. kt0+WD-2 and the last one tile kt0+WD-1.)
    load_codes(kt0, C[0]);
#pragma unroll
    for (int q = 0; q < XR; ++q) dma_x(&lds[0], kt0, q);
#pragma unroll
    for (int q = 0; q < XR; ++q) dma_x(&lds[XST], cl(kt0 + 1), q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 1; d + 1 < WD; ++d) load_codes(cl(kt0 + d), C[d]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < XR; ++q) dma_x(&lds[2 * XST], cl(kt0 + 2), q);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(cl(kt0 + WD - 1), C[WD - 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) table_unit(C[0], u);
#pragma unroll
    for (int w = 0; w < NUP; ++w) pair_unit(C[0], 0, w, Ap[0]);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((WD - 1) * LC + XR, 0));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < JT; ++j) op[0][j] = read_b(0, 0, j);

    // Hand-scheduled iteration.  Issue is in order, so back-to-back MFMAs
    // would hold everything behind them; instead each MFMA of the tile is
    // followed by a small, fixed amount of other work and a scheduling
    // fence, so the vector work executes while the matrix core is busy.
    // The stages are passed as restrict pointers: the ones read and the one
    // being filled are distinct, which lets the compiler leave the DMA in
    // flight across the reads.  The DMA's own completion is awaited by hand
    // (s_waitcnt) before the barrier that publishes a stage.
    auto iteration = [&](int64_t kt, auto phase, u32x4_t* __restrict__ rd0,
                         u32x4_t* __restrict__ rd1, u32x4_t* __restrict__ fill) {
      constexpr int ph = decltype(phase)::value;
      constexpr int SPK = NI * JT;  // MFMAs (slots) per k step
      constexpr int DP = 4 * SPK / XR;  // slots between the x DMAs (XR per tile)
      auto rb = [&](u32x4_t* st, int kk, int j) -> u32x4_t {
        return st[rk(32 * j + lr, 4 * lg + kk)];
      };
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // steps 0..2 decode pair kk+1 of this tile (NUP units); step 3
        // builds the next tile's table and decodes its pair 0 (8 + NUP)
        const int NU = kk < 3 ? NUP : 8 + NUP;
#pragma unroll
        for (int s = 0; s < SPK; ++s) {
          const int j = s / NI, i = s % NI;
          acc[i][j] = DT::mfma32(Ap[kk & 1][i], op[kk & 1][j], acc[i][j]);
          if (i == NI - 1) {
            // operand j of the next step: this tile's, or the next tile's
            // first (its stage was completed before the last barrier)
            if (kk < 3)
              op[(kk + 1) & 1][j] = rb(rd0, kk + 1, j);
            else
              op[0][j] = rb(rd1, 0, j);
          }
#pragma unroll
          for (int u = s * NU / SPK; u < (s + 1) * NU / SPK; ++u) {
            if (kk < 3)
              pair_unit(C[ph % WD], kk + 1, u, Ap[(kk + 1) & 1]);
            else if (u < 8)
              table_unit(C[(ph + 1) % WD], u);
            else
              pair_unit(C[(ph + 1) % WD], 0, u - 8, Ap[0]);
          }
          const int slot = SPK * kk + s;
          if (slot % DP == DP - 1) dma_x(fill, cl(kt + 3), slot / DP);  // x chunk of tile kt+3
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // tile kt's codes are consumed: tile kt+4's into their set, issued
      // after this iteration's DMA so that the wait below (for the x tile
      // DMA'd during the last iteration) does not also wait for them, nor
      // for the codes issued at the end of the last iteration: x tile kt+2
      // is complete once at most those LC + XR + LC loads are outstanding
      load_codes(cl(kt + WD), C[ph % WD]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(XR + 2 * LC, 0));
      __builtin_amdgcn_s_barrier();
    };
    u32x4_t* const S0 = &lds[0];
    u32x4_t* const S1 = &lds[XST];
    u32x4_t* const S2 = &lds[2 * XST];
    u32x4_t* const S3 = &lds[3 * XST];
    // Whole groups of four in the loop, the rest after it: the loop's back
    // edge then only ever follows phase 3, so the compiler's wait analysis
    // sees every load's true age at the loop head.
    int64_t kt = kt0;
    for (; kt + 4 <= kt1; kt += 4) {
      iteration(kt, std::integral_constant<int, 0>(), S0, S1, S3);
      iteration(kt + 1, std::integral_constant<int, 1>(), S1, S2, S0);
      iteration(kt + 2, std::integral_constant<int, 2>(), S2, S3, S1);
      iteration(kt + 3, std::integral_constant<int, 3>(), S3, S0, S2);
    }
    if (kt < kt1) {
      iteration(kt, std::integral_constant<int, 0>(), S0, S1, S3);
      if (kt + 1 < kt1) {
        iteration(kt + 1, std::integral_constant<int, 1>(), S1, S2, S0);
        if (kt + 2 < kt1) iteration(kt + 2, std::integral_constant<int, 2>(), S2, S3, S1);
      }
    }
    // the clamped prefetches past the split are still writing LDS
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  }

  // --- adapter columns: xs [M, 2r] against [B | B] (last split only) ---
  const int r = p.r;
  if (z == nz - 1) {
    const int ext_tiles = (2 * r + KT - 1) / KT;
    for (int e = 0; e < ext_tiles; ++e) {
      __syncthreads();  // the ring is free
#pragma unroll
      for (int q = 0; q < XR; ++q) {
        const int64_t m = clamp_row(m0 + (t >> 3) + 32 * q, M);
        const int col = e * KT + 8 * (t & 7);
        const u32x4_t v =
            col < 2 * r ? *reinterpret_cast<const u32x4_t*>(p.xs + m * 2 * r + col) : zero;
        store_x(0, q, v);
      }
      u32x4_t a[NI][4];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int64_t row = clamp_row(n0 + RW * wave + 32 * i + lr, N);
          const int col = e * KT + 8 * (4 * lg + kk);
          const int jj = col < r ? col : col - r;
          a[i][kk] = col < 2 * r ? *reinterpret_cast<const u32x4_t*>(p.B + row * r + jj) : zero;
        }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < JT; ++j) {
          const u32x4_t b = read_b(0, kk, j);
#pragma unroll
          for (int i = 0; i < NI; ++i) acc[i][j] = DT::mfma32(a[i][kk], b, acc[i][j]);
        }
    }
  }

  // --- epilogue: D[n][m] -> y[m][n], or the split's fp32 partial ---
  __syncthreads();  // the LDS ring is free from here on
  float* scratch = reinterpret_cast<float*>(&lds[0]) + wave * epi_floats<NI>();
  if (bw.tail >= 0)  // tile-local [TM][TN] partial
    store_acc_tile<NI, JT, DT>(acc, scratch, RW * wave, 0, N - n0, M - m0, true,
                               p.part + ((int64_t)z * p.tail_q + bw.tail) * TM * TN, nullptr,
                               TN, lane);
  else
    store_acc_tile<NI, JT, DT>(acc, scratch, n0 + RW * wave, m0, N, M, nz > 1,
                               nz > 1 ? p.part + (int64_t)z * M * N : nullptr, p.y, N, lane);
}

// out[i] = DT(sum_z part[z][i]), i over M*N (4 per thread), fixed order.
template <class DT>
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
    o[0] = DT::pack2(s[0], s[1]);
    o[1] = DT::pack2(s[2], s[3]);
    *reinterpret_cast<u32x2_t*>(out + i) = o;
  }
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t count, uint16_t* out,
                                hipStream_t s, bool f16) {
  int64_t g = (count / 4 + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  if (f16)
    hipLaunchKernelGGL(splitk_reduce_kernel<F16T>, dim3((unsigned)g), dim3(256), 0, s, part,
                       splits, count, out);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<Bf16T>, dim3((unsigned)g), dim3(256), 0, s, part,
                       splits, count, out);
  return hipGetLastError();
}

// Tail partials -> 16-bit output: out[m0 + mi][n0 + ni] = DT(sum_z
// tpart[z][q][mi][ni]) for the tail tiles q, fixed split order; 4 elements
// per thread.
template <class DT>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ tpart,
                                                          int tm, int64_t full, int tail_q,
                                                          int tail_s, int64_t M, int64_t Nout,
                                                          uint16_t* __restrict__ out) {
  const int64_t m_tiles = (M + tm - 1) / tm, n_tiles = (Nout + TILE_N - 1) / TILE_N;
  const int64_t per_tile = (int64_t)tm * TILE_N / 4;
  const int64_t count = per_tile * tail_q;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const int64_t q = i / per_tile, e = i - q * per_tile;
    const int64_t mi = e / (TILE_N / 4), ni = 4 * (e % (TILE_N / 4));
    int64_t mt, nt;
    tile_of_rank(full + q, m_tiles, n_tiles, 4, mt, nt);
    const int64_t m = mt * tm + mi, n = nt * TILE_N + ni;
    if (m >= M || n >= Nout) continue;
    const float* src = tpart + (q * tm + mi) * TILE_N + ni;
    f32x4_t sum = *reinterpret_cast<const f32x4_t*>(src);
    for (int z = 1; z < tail_s; ++z) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + (int64_t)z * tail_q * tm * TILE_N);
      sum[0] += v[0];
      sum[1] += v[1];
      sum[2] += v[2];
      sum[3] += v[3];
    }
    u32x2_t o;
    o[0] = DT::pack2(sum[0], sum[1]);
    o[1] = DT::pack2(sum[2], sum[3]);
    *reinterpret_cast<u32x2_t*>(out + m * Nout + n) = o;
  }
}

// Schedule of a fused GEMM: output Mout x Nout, reduction Kred (both GEMMs
// tile the reduction by 64 and the non-token output dimension by 256, or
// by 128 with the narrow tiles).  For
// each block tile the estimate is
//   rounds * (time of one tile on one CU) + fp32 partial traffic,
// where a round is 256 concurrent blocks (one per CU).  Few tiles: split
// every tile's reduction until ~256 blocks run (flops counted on the token
// rows the tiles cover, padding included).  Otherwise the tiles run whole,
// except that a last round filled less than half is split: its tail_q
// tiles are split 256 / tail_q ways (at most 8, at least 4 k tiles each),
// so it takes a fraction of a round.  The rates are the measured sustained
// throughputs of the tiles.  With `narrow` (a GEMM on the NF4 weight) a
// 128 x 128 tile is considered too, for the split schedule or for whole
// tiles that fill whole rounds (never the split tail).
GemmConfig gemm_config(int64_t M, int64_t Nout, int64_t Kred, bool narrow) {
  constexpr int kSlots = 256;  // concurrent blocks: one per CU
  const int64_t nkt = Kred / KT;
  GemmConfig best{256, 1, 0, 0, 1, TILE_N};
  double best_t = 1e300;
  struct Shape {
    int tm, tn;
    double rate;  // flop/s, whole chip
  };
  const Shape shapes[3] = {{256, TILE_N, 1.1e15}, {128, TILE_N, 0.8e15}, {128, 128, 0.85e15}};
  for (int si = 0; si < (narrow ? 3 : 2); ++si) {
    const int tm = shapes[si].tm, tn = shapes[si].tn;
    const double rate = shapes[si].rate;
    const int64_t m_t = (M + tm - 1) / tm;
    const int64_t tiles = m_t * ((Nout + tn - 1) / tn);
    const double t_tile = 2.0 * tm * tn * (double)Kred / (rate / kSlots);
    GemmConfig c{tm, 1, 0, 0, 1, tn};
    double est;
    if (tiles < 192) {
      int64_t sp = 256 / tiles;
      if (sp > nkt / 4) sp = nkt / 4;
      if (sp > 16) sp = 16;
      if (sp < 1) sp = 1;
      c.splits = (int)sp;
      const double blocks = (double)tiles * sp;
      const double fill = blocks >= kSlots ? 1.0 : blocks / kSlots;
      est = 2.0 * (m_t * tm) * Nout * (double)Kred / (rate * fill);
      if (sp > 1) est += 2.0 * sp * (double)M * Nout * 4 / 5.0e12;
    } else {
      const int64_t rounds = tiles / kSlots, q = tiles % kSlots;
      if (tn != TILE_N && q != 0) continue;
      int64_t ts = q > 0 ? kSlots / q : 1;
      if (ts > nkt / 4) ts = nkt / 4;
      if (ts > 8) ts = 8;
      if (q > 0 && ts >= 2) {
        c.full = tiles - q;
        c.tail_q = (int)q;
        c.tail_s = (int)ts;
        est = (rounds + 1.0 / ts) * t_tile + 2.0 * ts * q * tm * tn * 4 / 5.0e12;
      } else {
        est = (rounds + (q > 0 ? 1 : 0)) * t_tile;
      }
    }
    if (est < best_t) {
      best_t = est;
      best = c;
    }
  }
  return best;
}

int64_t gemm_blocks(const GemmConfig& c, int64_t M, int64_t Nout) {
  if (c.tail_q > 0) return c.full + (int64_t)c.tail_q * c.tail_s;
  return ((Nout + c.tn - 1) / c.tn) * ((M + c.tm - 1) / c.tm) * c.splits;
}

size_t gemm_partial_bytes(const GemmConfig& c, int64_t M, int64_t Nout) {
  if (c.tail_q > 0) return (size_t)c.tail_s * c.tail_q * c.tm * TILE_N * sizeof(float);
  if (c.splits > 1) return (size_t)c.splits * M * Nout * sizeof(float);
  return 0;
}

hipError_t launch_gemm_reduce(const GemmConfig& c, const float* part, int64_t M, int64_t Nout,
                              uint16_t* out, hipStream_t s, bool f16) {
  if (c.tail_q > 0) {
    const int64_t count = (int64_t)c.tail_q * c.tm * TILE_N / 4;
    int64_t g = (count + 255) / 256;
    if (g > 8192) g = 8192;
    if (f16)
      hipLaunchKernelGGL(tail_reduce_kernel<F16T>, dim3((unsigned)g), dim3(256), 0, s, part,
                         c.tm, c.full, c.tail_q, c.tail_s, M, Nout, out);
    else
      hipLaunchKernelGGL(tail_reduce_kernel<Bf16T>, dim3((unsigned)g), dim3(256), 0, s, part,
                         c.tm, c.full, c.tail_q, c.tail_s, M, Nout, out);
    return hipGetLastError();
  }
  if (c.splits > 1) return launch_splitk_reduce(part, c.splits, M * Nout, out, s, f16);
  return hipSuccess;
}

// block tile (tokens x n) and compute type for a weight format: fp16 and
// the narrow tile with the NF4 weight only
template <int WF>
static void launch_fwd_kernel(const GemmConfig& cfg, bool f16, dim3 grid, hipStream_t s,
                              const FwdParams& p) {
  constexpr bool Q = WF != kWeightBf16;
  if (cfg.tn != TILE_N) {
    if constexpr (Q) {
      if (f16)
        hipLaunchKernelGGL((fwd_gemm_kernel<4, WF, F16T, 32>), grid, dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL((fwd_gemm_kernel<4, WF, Bf16T, 32>), grid, dim3(256), 0, s, p);
    }
  } else if (cfg.tm == 256) {
    if constexpr (Q) {
      if (f16) {
        hipLaunchKernelGGL((fwd_gemm_kernel<8, WF, F16T, 64>), grid, dim3(256), 0, s, p);
        return;
      }
    }
    hipLaunchKernelGGL((fwd_gemm_kernel<8, WF, Bf16T, 64>), grid, dim3(256), 0, s, p);
  } else {
    if constexpr (Q) {
      if (f16) {
        hipLaunchKernelGGL((fwd_gemm_kernel<4, WF, F16T, 64>), grid, dim3(256), 0, s, p);
        return;
      }
    }
    hipLaunchKernelGGL((fwd_gemm_kernel<4, WF, Bf16T, 64>), grid, dim3(256), 0, s, p);
  }
}

hipError_t launch_fwd_gemm(const uint8_t* codes, const uint8_t* qscale, const float* step,
                           const float* dq_mean, const uint16_t* wbf, const uint16_t* x,
                           const uint16_t* xs, const uint16_t* B, uint16_t* y, float* part,
                           int64_t M, int64_t N,
                           int64_t K, int r, const Nf4Levels& L, hipStream_t s, bool f16) {
  const bool nf4 = wbf == nullptr;
  const GemmConfig cfg = gemm_config(M, N, K, nf4);
  if (gemm_partial_bytes(cfg, M, N) > 0 && part == nullptr) return hipErrorInvalidValue;
  FwdParams p;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.dq_mean = dq_mean;
  p.wbf = wbf;
  p.x = x;
  p.xs = xs;
  p.B = B;
  p.y = y;
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
  const int64_t blocks = gemm_blocks(cfg, M, N);
  const dim3 grid((unsigned)blocks);
  if (!nf4)
    launch_fwd_kernel<kWeightBf16>(cfg, false, grid, s, p);
  else if (dq_mean)
    launch_fwd_kernel<kWeightNf4Centred>(cfg, f16, grid, s, p);
  else
    launch_fwd_kernel<kWeightNf4>(cfg, f16, grid, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_reduce(cfg, part, M, N, y, s, f16);
}

}  // namespace qlora
