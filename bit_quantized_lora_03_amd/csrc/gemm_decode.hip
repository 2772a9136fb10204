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
//  * a block owns 32 weight rows over the whole reduction, so no partial
//    sums leave the chip: the row's NF4 blocks are dealt to 16 slots (8
//    waves x the two lane halves), lane (row l%32, half l/32) of wave w
//    taking slot 2 w + l/32 of each chunk of 16 blocks.  Each wave brings
//    in exactly the codes it decodes by DMA, into an LDS ring of its own
//    six chunks deep, so waves never wait for one another until the final
//    sum.  For each block the lane builds the block's 16-entry bf16
//    table once and decodes its 64 codes into the A operands of 8
//    consecutive MFMAs; the reduction order over k is permuted consistently
//    for A and B (MFMA j of a block pair sums k = 64 b + 8 j + e, e = 0..7,
//    over the two lane halves' blocks b);
//  * the table lives in LDS, entry c of lane l of wave w at byte
//    4096 w + 256 c + 4 l, so a lookup is one v_perm (which places the
//    code, tagged with the wave, next to the lane's byte offset) and one
//    2-byte LDS read, and the 64 lanes of a read always hit 64 distinct
//    banks -- about two thirds of the vector work of resolving codes with
//    byte permutes in registers;
//  * x is small and stays in L2: each token lane reads its 16-byte operand
//    pieces directly, two chunks ahead (lanes past the M tokens read
//    nothing: their offsets lie beyond x, which returns zeros);
//  * the 8 waves' partial tiles are added in LDS in wave order.
//
// The adapter's down projection x . A^T rides along: rows of A (bf16, used
// as they are) form extra 32-row tiles, split over k into short pieces
// (their partial sums land in columns N .. N+r-1 of part[z]).  Those tiles
// come last in the grid and fill in as the weight tiles finish.  With an adapter, the weight tiles write their fp32 sums to part[0]
// and decode_reduce forms the fp32 adapter term (alpha/r) . (x . A^T) . B^T
// and rounds y to bf16 once; without one, the weight tiles round and store
// y themselves.
//
// Grid: 1-D over the weight tiles, then (A tiles x SA splits).

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int WAVES = 8;    // waves per block
constexpr int SLOTS = 2 * WAVES;  // NF4-block slots per weight row
constexpr int SPAN = 128;   // k per span of the adapter tiles
constexpr int kTabBytes = WAVES * 16 * 64 * 4;  // per-lane NF4 tables, 32 KiB
constexpr int NSTAGE = 6;   // code chunks in the LDS ring
constexpr int kStageU4 = 32 * 64 / 16;  // one wave's chunk: 32 rows x its 2 blocks (64 bytes)
constexpr int kLdsBytes = kTabBytes + WAVES * NSTAGE * kStageU4 * 16;
constexpr int kXBytes = 32768;  // x staged in LDS when it fits (see decode_x_in_lds)

// s_waitcnt immediate: wait until at most `vm` vector-memory and `lgkm` LDS
// operations of this wave are outstanding (expcnt left free).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

struct DecodeParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* x;
  const uint16_t* A;
  float* part;
  int64_t M, N, K;
  int r;
  uint16_t* y;         // bf16 output when r == 0 (no adapter term to add)
  int sa;              // k splits of the A tiles
  int64_t w_blocks;    // weight tiles (they come first)
  int64_t blocks;      // w_blocks + A tiles x sa
  Nf4Levels L;
};

// codes of one NF4 block plus the raw scale byte and step: s' is formed
// only when the block is decoded, so that issuing the loads never waits
struct Blk {
  u32x4_t c[2];
  uint32_t q;
  float st;
};

}  // namespace

// XL: x lives in LDS for the whole reduction (few tokens; decode_x_in_lds)
template <bool XL>
__global__ __launch_bounds__(WAVES * 64) void decode_main_kernel(DecodeParams p) {
  // the tables start the kernel's LDS (at offset 0, so a lookup address
  // needs no base added); after the main loop the space holds the reduction
  __shared__ __align__(16) uint8_t lds[kLdsBytes + (XL ? kXBytes : 0)];

  // Weight tiles take the first ids, A tiles the last: workgroups are
  // dispatched in id order, so the A tiles fill in as weight tiles finish
  // instead of holding CUs the weight tiles need.  Among the weight tiles,
  // ids are turned into ranks contiguous within an XCD (ids are dealt to
  // the 8 XCDs round-robin), so neighbouring row tiles share an L2.
  const int64_t id = blockIdx.x;
  if (id >= p.blocks) return;
  const bool a_tile = id >= p.w_blocks;
  int64_t tile;
  int z = 0;
  if (a_tile) {
    tile = (id - p.w_blocks) / p.sa;
    z = (int)((id - p.w_blocks) % p.sa);
  } else {
    const int64_t xcd = id % 8, per = p.w_blocks / 8, extra = p.w_blocks % 8;
    tile = xcd * per + (xcd < extra ? xcd : extra) + id / 8;
  }

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t n0 = tile * 32;
  const int64_t nrows = a_tile ? p.r : N;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const int64_t n = n0 + lr;
  const bool row_ok = n < nrows;
  const bool tok_ok = lr < M;
  const uint16_t* xrow = p.x + (tok_ok ? lr : 0) * K;
  const __amdgpu_buffer_rsrc_t xres = make_rsrc(p.x, (uint32_t)(M * K * 2));

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  // x operands of the 64 k starting at kb (8 pieces of 16 bytes).  Lanes
  // past the M tokens read token 0's row (their columns of the product are
  // never stored): the loads are unconditional, so no branch makes the
  // compiler's wait analysis assume they might be missing.
  auto load_x = [&](int64_t kb, u32x4_t (&xb)[8]) {
    const uint16_t* xp = xrow + kb;
#pragma unroll
    for (int j = 0; j < 8; ++j) xb[j] = *reinterpret_cast<const u32x4_t*>(xp + 8 * j);
  };

  if (!a_tile) {
    // The row's NF4 blocks go in chunks of 16 (1024 k); within a chunk lane
    // (row l%32, half l/32) of wave w decodes block 2 w + l/32.  Each wave
    // brings in exactly the codes it decodes -- its two blocks of the 32
    // rows, 64 bytes per row and chunk -- by DMA (buffer loads that write
    // LDS directly) into a ring of its own, NSTAGE chunks deep, so no wave
    // waits for another: the main loop has no barrier.  (Together the 8
    // waves read each row's 512-byte chunk piece.)  In a stage, row r's
    // 16-byte piece p (0, 1: block 2 w; 2, 3: block 2 w + 1) sits at
    // r * 64 + 16 (p ^ ((r / 4) % 4)), so the 16 rows one LDS read cycle
    // serves cover all 64 banks.  Scale bytes, steps and x pieces are
    // per-lane loads into registers.
    const int64_t nblk = K / 64;
    const int64_t nch = (nblk + 15) / 16;
    const int slot = 2 * wave + lg;
    const int64_t row_blk = ((row_ok ? n : 0) * K) >> 6;
    const __amdgpu_buffer_rsrc_t cres = make_rsrc(p.codes, (uint32_t)((N * K) >> 1));
    uint32_t cvoff[2];  // instruction h fills physical pieces 64 h + lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pc = 64 * h + lane, r = pc >> 2;
      const int lp = (pc & 3) ^ ((r >> 2) & 3);
      cvoff[h] = (uint32_t)((n0 + r) * (K >> 1) + 64 * wave + 16 * lp);
    }
    auto dma_codes = [&](u32x4_t* stage, int64_t ch) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            cres, (__attribute__((address_space(3))) void*)(stage + 64 * h), 16,
            cvoff[h] + (uint32_t)(ch * 512), 0, 0, 0);
    };
    struct Scale {
      uint32_t q;
      float st;
    };
    auto blk_of = [&](int64_t ch) { return 16 * ch + slot; };
    auto load_scale = [&](int64_t ch, Scale& S) {
      const int64_t b = blk_of(ch) < nblk ? blk_of(ch) : 0;
      S.q = p.qscale[row_blk + b];
      S.st = p.step[(row_blk + b) >> 8];
    };
    // x pieces of the lane's block of chunk ch: 8 x 16 bytes of token lr.
    // Lanes past the M tokens (and blocks past the row's end) get a lane
    // offset beyond x, so their loads return zero without touching memory;
    // the loads themselves are unconditional, so no branch makes the
    // compiler's wait analysis assume they might be missing.
    const uint32_t xrow_off = (uint32_t)(lr * K * 2);
    auto load_xc = [&](int64_t ch, u32x4_t (&xb)[8]) {
      const uint32_t off = (tok_ok && blk_of(ch) < nblk)
                               ? xrow_off + (uint32_t)(blk_of(ch) * 128)
                               : 0x80000000u;
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[j] = buffer_load16(xres, off + 16 * j);
    };

    uint16_t* tab_w = reinterpret_cast<uint16_t*>(lds) + wave * 2048 + lane * 2;
    const uint32_t wtag = (uint32_t)wave * 0x10101010u;  // wave in bits 4..7 of each code byte
    const uint32_t lane4 = (uint32_t)lane * 4u;
    const int rsw = (lr >> 2) & 3;
    auto decode_chunk = [&](const u32x4_t* stage, int64_t ch, const Scale& S, auto&& xop) {
      const bool ok = row_ok && blk_of(ch) < nblk;
      const u32x4_t c0 = stage[lr * 4 + ((2 * lg) ^ rsw)];
      const u32x4_t c1 = stage[lr * 4 + ((2 * lg + 1) ^ rsw)];
      // this lane's block table: entry c = bf16_rne(fp32(L[c] * s'))
      const float sc = ok ? nf4_block_scale(S.q, S.st) : 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t pk = pack_bf16x2(p.L.v[2 * q] * sc, p.L.v[2 * q + 1] * sc);
        tab_w[(2 * q) * 128] = (uint16_t)pk;
        tab_w[(2 * q + 1) * 128] = (uint16_t)(pk >> 16);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t v = (j < 4 ? c0 : c1)[j & 3];
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
        acc = mfma32x32x16(a, xop(j), acc);
      }
    };

    // Issue order.  The prologue loads x (of chunks 0 and 1, or -- with x
    // in LDS -- every piece of x the wave will read), then the DMA and
    // scales of chunks 0 .. NSTAGE - 2; iteration ch loads x of chunk
    // ch + 2 (not with x in LDS), then issues the DMA of chunk
    // ch + NSTAGE - 1 and its scales, decodes chunk ch and at its end waits
    // for chunk ch + 1's DMA.  Loads complete in order, so a wait for x of
    // chunk ch (issued first in iteration ch - 2) also waits for the DMAs
    // issued before it, up to chunk ch + 2's: x comes two iterations ahead
    // and first in its iteration so that this never forces a DMA earlier
    // than three iterations after its issue (x in LDS takes x out of the
    // count altogether).  The end-of-iteration wait is "at most W
    // outstanding", W being the number of operations issued after chunk
    // ch + 1's DMA; with kOps operations per iteration that is
    // 2 + kOps (NSTAGE - 2) in the steady state (it was issued in iteration
    // ch + 2 - NSTAGE) and, with x in registers, 26 + 8 ch while the DMA
    // came from the prologue.  Waits are immediates, so W is a template
    // argument: the first group of iterations gets its own, later groups the
    // steady one, and a short reduction (fewer chunks than one group) the
    // smallest, which waits at least as long as needed.
    constexpr int kOps = XL ? 4 : 12;  // vector-memory operations per iteration
    constexpr int kWaitSteady = 2 + kOps * (NSTAGE - 2);
    static_assert(kWaitSteady <= 63, "vmcnt holds at most 63");
    u32x4_t* const ring =
        reinterpret_cast<u32x4_t*>(lds + kTabBytes) + wave * NSTAGE * kStageU4;
    Scale Sc[NSTAGE];
    u32x4_t X[XL ? 1 : 3][8];
    const int64_t lastc = nch - 1;
    auto cl = [&](int64_t c) { return c < lastc ? c : lastc; };

    // x in LDS: rows of 2K + 16 bytes (the pad puts consecutive tokens 4
    // banks apart), then one 128-byte zero area per wave, read by lanes
    // past the M tokens and for blocks past the row's end.  Each wave
    // stages exactly the pieces it reads -- its two blocks of every chunk,
    // for every token -- so no other wave's writes are involved: piece
    // i = lane + 64 q is byte 16 (i mod 16) of block 16 ch + 2 w + (i mod
    // 16) / 8, chunk ch = (i / 16) mod nch, token (i / 16) / nch.
    uint8_t* const xl = lds + kLdsBytes;
    const int64_t xrb = 2 * K + 16;
    constexpr int kXq = 4;  // pieces per lane (the x budget bounds M K / 64 by 256)
    u32x4_t xv[XL ? kXq : 1];
    uint32_t xdst[XL ? kXq : 1];
    if constexpr (XL) {
      // 32-bit index math, every offset computed before the select, so the
      // selects stay selects (a branch around the loads would make the
      // compiler wait for each load before the next)
      const uint32_t nch32 = (uint32_t)nch, m32 = (uint32_t)M, nblk32 = (uint32_t)nblk;
      const uint32_t xrow_bytes = (uint32_t)(2 * K), xrb32 = (uint32_t)xrb;
#pragma unroll
      for (int q = 0; q < kXq; ++q) {
        const uint32_t i = (uint32_t)(lane + 64 * q);
        const uint32_t pc = i & 15u, rest = i >> 4;
        const uint32_t tk = rest / nch32, c = rest - tk * nch32;
        const uint32_t b = 16u * c + 2u * (uint32_t)wave + (pc >> 3);
        const uint32_t col = 128u * b + 16u * (pc & 7u);
        const bool ok = tk < m32 && b < nblk32;
        const uint32_t src = tk * xrow_bytes + col, dst = tk * xrb32 + col;
        xv[q] = buffer_load16(xres, ok ? src : 0x80000000u);
        xdst[q] = ok ? dst : 0xFFFFFFFFu;
      }
    } else {
      load_xc(0, X[0]);
      load_xc(cl(1), X[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NSTAGE - 1; ++c) {
      dma_codes(ring + c * kStageU4, cl(c));
      load_scale(cl(c), Sc[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (XL) {
      // the wave's own pieces and zero area; its later reads follow in order
#pragma unroll
      for (int q = 0; q < kXq; ++q)
        if (xdst[q] != 0xFFFFFFFFu) *reinterpret_cast<u32x4_t*>(xl + xdst[q]) = xv[q];
      if (lane < 8) *reinterpret_cast<u32x4_t*>(xl + M * xrb + 128 * wave + 16 * lane) = zero;
    }
    // chunk 0's DMA: followed by its scales and NSTAGE - 2 DMA + scale pairs
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 + 4 * (NSTAGE - 2), 0));

    // x operand j of chunk ch from LDS: token lr's 16 bytes at k = 64 b + 8 j
    auto x_lds = [&](int64_t ch) {
      const int64_t b = blk_of(ch);
      const uint32_t xa = (tok_ok && b < nblk) ? (uint32_t)(lr * xrb + 128 * b)
                                                : (uint32_t)(M * xrb + 128 * wave);
      return [=](int j) -> u32x4_t {
        return *reinterpret_cast<const u32x4_t*>(xl + xa + 16 * j);
      };
    };

    // phase = ch mod NSTAGE: the stage read (rd), the stage filled (fill),
    // the scale set and the x set (ch mod 3) are then compile-time choices
    auto iteration = [&](int64_t ch, auto phase, auto wait, const u32x4_t* __restrict__ rd,
                         u32x4_t* __restrict__ fill) {
      constexpr int ph = decltype(phase)::value;
      constexpr int W = decltype(wait)::value;
      static_assert(NSTAGE % 3 == 0, "x sets rotate with the phase");
      if constexpr (!XL) {
        load_xc(cl(ch + 2), X[(ph + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
      dma_codes(fill, cl(ch + NSTAGE - 1));
      load_scale(cl(ch + NSTAGE - 1), Sc[(ph + NSTAGE - 1) % NSTAGE]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (XL)
        decode_chunk(rd, ch, Sc[ph], x_lds(ch));
      else
        decode_chunk(rd, ch, Sc[ph], [&](int j) -> u32x4_t { return X[ph % 3][j]; });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(W, 0));
    };
    static_assert(NSTAGE == 6, "the loop below is unrolled for six stages");
    u32x4_t* const R[NSTAGE] = {ring, ring + kStageU4, ring + 2 * kStageU4,
                                ring + 3 * kStageU4, ring + 4 * kStageU4, ring + 5 * kStageU4};
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using P4 = std::integral_constant<int, 4>;
    using P5 = std::integral_constant<int, 5>;
    // with x in LDS every iteration's count is the steady one
    using W0 = std::integral_constant<int, XL ? kWaitSteady : 26>;
    using W1 = std::integral_constant<int, XL ? kWaitSteady : 34>;
    using W2 = std::integral_constant<int, XL ? kWaitSteady : 42>;
    using WS = std::integral_constant<int, kWaitSteady>;
    static_assert(XL || 26 + 8 * (NSTAGE - 3) == kWaitSteady,
                  "iteration NSTAGE - 3 reaches the steady state");
    if (nch >= 6) {
      iteration(0, P0(), W0(), R[0], R[5]);
      iteration(1, P1(), W1(), R[1], R[0]);
      iteration(2, P2(), W2(), R[2], R[1]);
      iteration(3, P3(), WS(), R[3], R[2]);
      iteration(4, P4(), WS(), R[4], R[3]);
      iteration(5, P5(), WS(), R[5], R[4]);
      int64_t ch = 6;
      for (; ch + 6 <= nch; ch += 6) {
        iteration(ch, P0(), WS(), R[0], R[5]);
        iteration(ch + 1, P1(), WS(), R[1], R[0]);
        iteration(ch + 2, P2(), WS(), R[2], R[1]);
        iteration(ch + 3, P3(), WS(), R[3], R[2]);
        iteration(ch + 4, P4(), WS(), R[4], R[3]);
        iteration(ch + 5, P5(), WS(), R[5], R[4]);
      }
      if (ch < nch) iteration(ch, P0(), WS(), R[0], R[5]);
      if (ch + 1 < nch) iteration(ch + 1, P1(), WS(), R[1], R[0]);
      if (ch + 2 < nch) iteration(ch + 2, P2(), WS(), R[2], R[1]);
      if (ch + 3 < nch) iteration(ch + 3, P3(), WS(), R[3], R[2]);
      if (ch + 4 < nch) iteration(ch + 4, P4(), WS(), R[4], R[3]);
    } else {
      iteration(0, P0(), W0(), R[0], R[5]);
      if (1 < nch) iteration(1, P1(), W0(), R[1], R[0]);
      if (2 < nch) iteration(2, P2(), W0(), R[2], R[1]);
      if (3 < nch) iteration(3, P3(), W0(), R[3], R[2]);
      if (4 < nch) iteration(4, P4(), W0(), R[4], R[3]);
    }
    // the clamped prefetches past the end are still writing LDS
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  } else {
    // rows of A: bf16 operands as stored; this split's spans, cut in
    // contiguous pieces over the waves (k = span base + 64 lg + 8 j + e)
    const int64_t spans_total = (K + SPAN - 1) / SPAN;
    const int64_t bs0 = spans_total * z / p.sa, bs1 = spans_total * (z + 1) / p.sa;
    const int64_t per_w = (bs1 - bs0 + WAVES - 1) / WAVES;
    const int64_t s_begin = bs0 + wave * per_w < bs1 ? bs0 + wave * per_w : bs1;
    const int64_t s_end = s_begin + per_w < bs1 ? s_begin + per_w : bs1;
    const uint16_t* arow = p.A + (row_ok ? n : 0) * K;
    for (int64_t sp = s_begin; sp < s_end; ++sp) {
      const int64_t kb = sp * SPAN + 64 * lg;
      const bool ok = row_ok && kb < K;
      u32x4_t xb[8], av[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xb[j] = zero;
      load_x(kb < K ? kb : 0, xb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        av[j] = ok ? *reinterpret_cast<const u32x4_t*>(arow + kb + 8 * j) : zero;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = mfma32x32x16(av[j], xb[j], acc);
    }
  }

  // ---- sum the waves' tiles in LDS (wave order), write the result ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [WAVES][32 rows][M], M <= 32
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
      if (p.y)  // no adapter: this is y
        p.y[(int64_t)m * N + n0 + row] = __builtin_bit_cast(uint16_t, (__bf16)s);
      else
        p.part[((int64_t)z * M + m) * ldp + col0 + row] = s;
    }
  }
}

// y[m][n] = bf16( part[0][m][n] + scale * sum_j xa[m][j] B[n][j] ) with
// xa[m][j] = sum_z part[z][m][N + j] (z < sa), fixed summation orders.
// The r-sum is a small matrix product, so it runs on MFMA like the fused
// GEMMs' adapter columns: xa is split into bf16 hi + lo (hi + lo equals the
// fp32 value to 2^-17), tokens as the 32 A rows, and B's rows -- 16-byte
// pieces along j, as stored -- as the B columns.  Block of 256 threads, 128
// columns n (32 per wave); the block first forms xa's hi/lo rows in LDS
// (every block does: xa is M x r), with all of a pass's loads issued before
// any is used.  Each lane's B pieces and base sums are loaded at the start,
// so their latency overlaps that phase.  Loads go through buffer
// descriptors (out-of-range offsets read zero), so no branch separates them.
constexpr int kMaxASplits = 16;
constexpr int kRedCols = 128;                   // columns per block
constexpr int kXsRow = 256 + 8;  // LDS row of xa's hi or lo (bf16): r <= 256 + 16 bytes of pad
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part,
                                                            int sa,
                                                            const uint16_t* __restrict__ B,
                                                            int r, float scale,
                                                            uint16_t* __restrict__ y, int64_t M,
                                                            int64_t N) {
  __shared__ __align__(16) uint16_t xs[2][kDecodeMaxM][kXsRow];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lr = lane & 31, lg = lane >> 5;
  const int64_t ldp = N + r;
  const int64_t n = (int64_t)blockIdx.x * kRedCols + 32 * wave + lr;  // this lane's column
  const bool n_ok = n < N;
  const int ks = (r + 15) / 16;                   // 16-wide MFMA steps over j
  constexpr uint32_t kOut = 0x80000000u;          // past both tensors
  const __amdgpu_buffer_rsrc_t pres =
      make_rsrc(part, (uint32_t)((int64_t)sa * M * ldp * 4));
  const __amdgpu_buffer_rsrc_t bres = make_rsrc(B, (uint32_t)(N * r * 2));

  // B operand of step s: B[n][16 s + 8 lg .. + 7]
  constexpr int kMaxSteps = 256 / 16;  // r <= 256
  u32x4_t bop[kMaxSteps];
#pragma unroll
  for (int s2 = 0; s2 < kMaxSteps; ++s2) {
    const int j = 16 * s2 + 8 * lg;
    bop[s2] = buffer_load16(bres, (n_ok && j < r) ? (uint32_t)((n * r + j) * 2) : kOut);
  }
  // base sums of the tokens this lane's accumulators hold:
  // rows 8 (v / 4) + 4 lg + v % 4 of the 32 x 32 tile
  float base[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t m = 8 * (v >> 2) + 4 * lg + (v & 3);
    base[v] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   pres, (n_ok && m < M) ? (int)((m * ldp + n) * 4) : (int)kOut, 0, 0));
  }

  // xa's hi/lo rows for tokens < M (j < 16 ks; zero past r), 4 per thread per pass
  constexpr int EPT = 4;
  const int cols = 16 * ks;
  const int total = (int)M * cols;
  for (int e0 = t; e0 < total; e0 += 256 * EPT) {
    float v[EPT][kMaxASplits];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = e0 + 256 * u;
      const int m = e / cols, j = e - m * cols;
      const uint32_t off = (uint32_t)(((int64_t)m * ldp + N + j) * 4);
#pragma unroll
      for (int z = 0; z < kMaxASplits; ++z) {
        const bool ok = e < total && j < r && z < sa;
        v[u][z] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       pres, ok ? (int)(off + (uint32_t)((int64_t)z * M * ldp * 4)) : (int)kOut,
                       0, 0));
      }
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = e0 + 256 * u;
      float acc = v[u][0];
#pragma unroll
      for (int z = 1; z < kMaxASplits; ++z)
        if (z < sa) acc += v[u][z];
      if (e < total) {
        const int m = e / cols, j = e - m * cols;
        const uint16_t hi = __builtin_bit_cast(uint16_t, (__bf16)acc);
        const uint16_t lo = __builtin_bit_cast(uint16_t, (__bf16)(acc - bf16_bits_to_f32(hi)));
        xs[0][m][j] = hi;
        xs[1][m][j] = lo;
      }
    }
  }
  // token rows past M are zero
  for (int e = (int)M * cols + t; e < kDecodeMaxM * cols; e += 256) {
    const int m = e / cols, j = e - m * cols;
    xs[0][m][j] = 0;
    xs[1][m][j] = 0;
  }
  __syncthreads();

  // D[token][n] = sum_j xa[token][j] B[n][j]: A = xa rows (lane: token lr,
  // j = 16 s + 8 lg ..), B = this lane's B pieces; hi, then lo, per step
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int s2 = 0; s2 < kMaxSteps; ++s2) {
    if (s2 < ks) {
      const u32x4_t ahi = *reinterpret_cast<const u32x4_t*>(&xs[0][lr][16 * s2 + 8 * lg]);
      const u32x4_t alo = *reinterpret_cast<const u32x4_t*>(&xs[1][lr][16 * s2 + 8 * lg]);
      acc = mfma32x32x16(ahi, bop[s2], acc);
      acc = mfma32x32x16(alo, bop[s2], acc);
    }
  }
  if (n_ok) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = 8 * (v >> 2) + 4 * lg + (v & 3);
      if (m < M)
        y[m * N + n] = __builtin_bit_cast(uint16_t, (__bf16)(base[v] + scale * acc[v]));
    }
  }
}

namespace {

// k splits of the adapter's A tiles, which run after the weight tiles as
// CUs free up: pieces of about 512 k (at most 16, the planes the reduction
// reads), so each takes about one memory round trip
int a_splits(int64_t K) {
  int64_t s = K / 512;
  if (s > kMaxASplits) s = kMaxASplits;
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace

// x fits in LDS: M rows of 2K + 16 bytes plus the waves' zero areas, and
// each wave's share (M tokens x its 16 pieces of every chunk) is at most
// 4 pieces per lane.
bool decode_x_in_lds(int64_t M, int64_t K) {
  const int64_t nch = (K / 64 + 15) / 16;
  return M * (2 * K + 16) + WAVES * 128 <= kXBytes && M * nch * 16 <= 64 * 4;
}

int decode_splits(int64_t M, int64_t N, int64_t K, int r) {
  (void)M;
  (void)N;
  return r > 0 ? a_splits(K) : 0;
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
  p.sa = r > 0 ? a_splits(K) : 1;
  if (r > 0 && (p.sa > splits || part == nullptr)) return hipErrorInvalidValue;
  p.y = r > 0 ? nullptr : y;
  p.w_blocks = (N + 31) / 32;
  p.blocks = p.w_blocks + (r > 0 ? (int64_t)((r + 31) / 32) * p.sa : 0);
  p.L = L;
  if (decode_x_in_lds(M, K))
    hipLaunchKernelGGL(decode_main_kernel<true>, dim3((unsigned)p.blocks), dim3(WAVES * 64), 0, s,
                       p);
  else
    hipLaunchKernelGGL(decode_main_kernel<false>, dim3((unsigned)p.blocks), dim3(WAVES * 64), 0, s,
                       p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || r == 0) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((N + kRedCols - 1) / kRedCols)),
                     dim3(256), 0, s, part, p.sa, B, r, scale, y, M, N);
  return hipGetLastError();
}

}  // namespace qlora
