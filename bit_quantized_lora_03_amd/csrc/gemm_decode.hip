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
//    (six chunks deep, three when x is staged in LDS, with the DMA three or
//    two chunks ahead), so waves never wait for one another until the final
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
//  * x is small and stays in L2.  When M rows of it fit in LDS each wave
//    stages, once, the pieces it will read; for up to 16 tokens each chunk's
//    pieces reach a two-stage ring of each wave by DMA, one chunk ahead
//    (four 1 KiB instructions per chunk instead of eight half-empty 16-byte
//    loads per lane, which the memory pipeline accepts at half the rate);
//    otherwise each token lane reads its 16-byte operand pieces directly,
//    two chunks ahead (lanes past the M tokens read nothing: their offsets
//    lie beyond x, which returns zeros);
//  * the 8 waves' partial tiles are added in LDS in wave order.
//
// The adapter's down projection x . A^T runs first, as a launch of the same
// kernel with only A tiles: rows of A (bf16, used as they are) form 32-row
// tiles, split over k into short pieces whose fp32 partial sums land in
// part[z][m][j].  The weight tiles then add the adapter term in their
// epilogue: xa = sum_z part[z] (split order), (alpha/r) . xa . B^T for the
// tile's 32 rows in fp32, and y is rounded to bf16 once.  Without an
// adapter only the weight launch runs.
//
// Grid: 1-D over the weight tiles (or, in the first launch, over the A
// tiles x SA splits).

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int WAVES = 8;    // waves per block
constexpr int SLOTS = 2 * WAVES;  // NF4-block slots per weight row
constexpr int SPAN = 128;   // k per span of the adapter tiles
constexpr int kTabBytes = WAVES * 16 * 64 * 4;  // per-lane NF4 tables, 32 KiB
// Code chunks in each wave's LDS ring, and chunks whose DMA is in flight
// ahead of the decode, with x in registers and with x in LDS.
constexpr int NSTAGE = 6, kAheadReg = 3;
constexpr int NSTAGE_XL = 3, kAheadXl = 2;
constexpr int kStageU4 = 32 * 64 / 16;  // one wave's chunk: 32 rows x its 2 blocks (64 bytes)
constexpr int ring_bytes(int nst) { return WAVES * nst * kStageU4 * 16; }
// x staged in LDS when it fits (see decode_x_in_lds): the rest of the 160 KiB
constexpr int kXBytes = 160 * 1024 - kTabBytes - ring_bytes(NSTAGE_XL);
constexpr int kXq = 8;  // x pieces each lane stages (bounds M K / 64 by 64 kXq)
// x by DMA per chunk (few tokens, x too large to stage whole): each wave's
// ring of two chunk stages, 16 tokens x its 2 blocks (256 bytes) each
constexpr int kXdTok = 16;
constexpr int kXdStage = kXdTok * 256;
constexpr int kXdBytes = WAVES * 2 * kXdStage;
// at most this many k splits of the A tiles (partial planes of x . A^T)
constexpr int kMaxASplits = 16;

// s_waitcnt immediate: wait until at most `vm` vector-memory and `lgkm` LDS
// operations of this wave are outstanding (expcnt left free).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

struct DecodeParams {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const float* dq_mean;  // the mean-centred scale format's mean (or null)
  const uint16_t* x;
  const uint16_t* A;
  const uint16_t* B;
  float* part;         // x . A^T partials [sa][M][r] fp32 (the A tiles' output)
  int64_t M, N, K;
  int r;
  float scale;         // alpha / r
  uint16_t* y;         // bf16 output of the weight tiles
  int sa;              // k splits of the A tiles
  const uint8_t* keep; // LoRA dropout keep mask [M, K / 8] on x . A^T's x (or null)
  PhiloxDrop drop;     // ... or keep bits drawn from Philox4x32-10 (rng != 0)
  int rng;
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

// XM: where x comes from.  1 (XL): x lives in LDS for the whole reduction
// (few tokens; decode_x_in_lds); 2 (XD): each chunk's x reaches a two-stage
// LDS ring of each wave by DMA, one chunk ahead (M <= kXdTok); 0: each
// token lane loads its x pieces into registers, two chunks ahead.
// CTR: the weight has the mean-centred scale format
template <int XM, bool CTR>
__global__ __launch_bounds__(WAVES * 64) void decode_main_kernel(DecodeParams p) {
  constexpr bool XL = XM == 1, XD = XM == 2;
  // the tables start the kernel's LDS (at offset 0, so a lookup address
  // needs no base added); after the main loop the space holds the reduction
  constexpr int NST = XL || XD ? NSTAGE_XL : NSTAGE;
  constexpr int kAhead = XL || XD ? kAheadXl : kAheadReg;
  static_assert(kAhead >= 2 && kAhead < NST, "prefetch distance within the ring");
  constexpr int kLdsBytes = kTabBytes + ring_bytes(NST);
  __shared__ __align__(16) uint8_t lds[kLdsBytes + (XL ? kXBytes : XD ? kXdBytes : 0)];

  // Weight tiles take the first ids, A tiles the rest (a launch holds one
  // kind or the other).  Among the weight tiles, ids are turned into ranks
  // contiguous within an XCD (ids are dealt to the 8 XCDs round-robin), so
  // neighbouring row tiles share an L2.
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
  const ScaleFmt fmt = scale_fmt(CTR ? p.dq_mean : nullptr);
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
    // LDS directly) into a ring of its own, NST chunks deep, so no wave
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
      const float sc =
          ok ? (CTR ? nf4_block_scale(S.q, S.st, fmt) : nf4_block_scale(S.q, S.st)) : 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t pk = pack_bf16x2(p.L.v[2 * q] * sc, p.L.v[2 * q + 1] * sc);
        tab_w[(2 * q) * 128] = (uint16_t)pk;
        tab_w[(2 * q + 1) * 128] = (uint16_t)(pk >> 16);
      }
      // the 8 table reads of step j (weights 8 j .. 8 j + 7 of the block)
      auto lookup = [&](int j, uint32_t (&h)[8]) {
        const uint32_t v = (j < 4 ? c0 : c1)[j & 3];
        // byte i of ev holds code 2i, of od code 2i + 1, each tagged with
        // 16 * wave; the address perm takes the byte straight from them
        const uint32_t ev = (v & 0x0F0F0F0Fu) | wtag;
        const uint32_t od = ((v >> 4) & 0x0F0F0F0Fu) | wtag;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // byte 0: the lane's offset, byte 1: code + 16 wave -> LDS address
          const uint32_t addr =
              perm((e & 1) ? od : ev, lane4, 0x0C0C0000u | ((4u + (e >> 1)) << 8));
          h[e] = *reinterpret_cast<const uint16_t*>(lds + addr);
        }
      };
      // Software-pipelined: step j + 1's reads are issued before step j's
      // values are packed, so each step's LDS latency runs behind the
      // previous step's packing and MFMA instead of stalling the wave.
      // (x operands read from LDS are issued with their step's lookups, so
      // waiting for a step's operands never waits for the next step's reads)
      uint32_t h[2][8];
      u32x4_t xv[2];
      lookup(0, h[0]);
      xv[0] = xop(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j + 1 < 8) {
          lookup(j + 1, h[(j + 1) & 1]);
          xv[(j + 1) & 1] = xop(j + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        u32x4_t a;
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = h[j & 1][2 * q] | (h[j & 1][2 * q + 1] << 16);
        acc = mfma32x32x16(a, xv[j & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Issue order.  The prologue issues, in rounds c = 0 .. kAhead - 1,
    // chunk c's DMA and scales, followed in round 0 by x of chunk 0 (or --
    // with x in LDS -- every piece of x the wave will read) and in round 1
    // by x of chunk 1; iteration ch loads x of chunk
    // ch + 2 (not with x in LDS), then issues the DMA of chunk
    // ch + kAhead and its scales, decodes chunk ch and at its end waits
    // for chunk ch + 1's DMA.  Loads complete in order, so a wait for x of
    // chunk ch (issued first in iteration ch - 2) also waits for the DMAs
    // issued before it, up to chunk ch + 2's: x comes two iterations ahead
    // and first in its iteration so that this never forces a DMA earlier
    // than three iterations after its issue (x in LDS takes x out of the
    // count altogether).  The end-of-iteration wait is "at most W
    // outstanding", W being the number of operations issued after chunk
    // ch + 1's DMA; with kOps operations per iteration that is
    // 2 + kOps (kAhead - 1) in the steady state (it was issued in iteration
    // ch + 1 - kAhead), and while chunk ch + 1 still comes from the
    // prologue, its scales, the prologue rounds after it (with x of chunk 1
    // after chunk 1's DMA when x is in registers) and iterations 0 .. ch
    // (wait_for below).  Waits are immediates, so W is a template
    // argument: the first group of iterations gets its own, later groups the
    // steady one, and a short reduction (fewer chunks than one group) the
    // smallest, which waits at least as long as needed.  The prefetch
    // distance is shorter than the ring: issued all at once, a deep
    // prologue holds every wave at the issue of its last loads (the CU's
    // request queue is full) for about as long as the chip takes to deliver
    // them, while chunk 0 is already there to decode.
    constexpr int kOps = XL ? 4 : XD ? 8 : 12;  // vector-memory operations per iteration
    // (XD: iteration ch issues x of chunk ch + 1 first, so the wait at its
    // end is for that x DMA -- and with it every earlier load -- leaving
    // only the iteration's code DMA and scales outstanding)
    constexpr int kWaitSteady = XD ? 4 : 2 + kOps * (kAhead - 1);
    static_assert(kWaitSteady <= 63, "vmcnt holds at most 63");
    // operations issued after chunk c + 1's DMA by the end of iteration c
    constexpr auto wait_for = [](int c) {
      if (XD || c + 1 >= kAhead) return kWaitSteady;
      return 2 + (!XL && c == 0 ? 8 : 0) + 4 * (kAhead - 2 - c) + kOps * (c + 1);
    };
    u32x4_t* const ring =
        reinterpret_cast<u32x4_t*>(lds + kTabBytes) + wave * NST * kStageU4;
    Scale Sc[NST];
    u32x4_t X[XL || XD ? 1 : 3][8];
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
    // XD: stage s of wave w at xl + kXdStage (2 w + s); token t's 256 bytes
    // (its 2 blocks of the chunk) at 256 t, logical 16-byte piece lp (block
    // lp / 8, piece lp % 8) at physical piece lp ^ t, so the 16 tokens one
    // 128-bit read cycle serves hit 16 distinct bank groups.  DMA
    // instruction q fills tokens 4 q .. 4 q + 3 (lane i: token 4 q + i / 16,
    // physical piece i % 16); tokens past M and blocks past the row's end
    // read zeros through an offset beyond x.
    uint8_t* const xdr = xl + (XD ? kXdStage * 2 * wave : 0);
    uint32_t xdoff[4];
    int xdblk[4];
    bool xdtok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tk = 4 * q + (lane >> 4), lp = (lane & 15) ^ tk;
      xdblk[q] = 2 * wave + (lp >> 3);
      xdtok[q] = tk < M;
      xdoff[q] = (uint32_t)(tk * K * 2 + 128 * xdblk[q] + 16 * (lp & 7));
    }
    auto dma_x = [&](uint8_t* stage, int64_t ch) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = xdtok[q] && 16 * ch + xdblk[q] < nblk;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)(stage + 1024 * q), 16,
            ok ? xdoff[q] + (uint32_t)(ch * 2048) : 0x80000000u, 0, 0, 0);
      }
    };
    // x operand j of a chunk in XD stage st: token lr % 16 (lanes of tokens
    // past 16 read a copy; their columns are never stored), block lg
    auto x_ring = [&](const uint8_t* st) {
      const int tk = lr & 15;
      const uint8_t* base = st + 256 * tk;
      return [=](int j) -> u32x4_t {
        return *reinterpret_cast<const u32x4_t*>(base + 16 * ((8 * lg + j) ^ tk));
      };
    };
    u32x4_t xv[XL ? kXq : 1];
    uint32_t xdst[XL ? kXq : 1];
    // The prologue's loads go out in rounds, one chunk per wave per round
    // with a barrier (issue order only: no memory is waited for) between
    // rounds, so every wave's chunk 0 reaches the memory pipeline before
    // any wave's chunk 1: issued wave by wave instead, the last waves'
    // first chunk queued behind the first waves' whole prefetch and landed
    // several microseconds later.  Round c: chunk c's DMA and scales, then
    // x (chunks 0 and 1 in registers, or every staged piece in round 0).
    if constexpr (XD) {
      dma_x(xdr, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < kAhead; ++c) {
      dma_codes(ring + c * kStageU4, cl(c));
      load_scale(cl(c), Sc[c]);
      if constexpr (XD) {
      } else if constexpr (XL) {
        if (c == 0) {
          // 32-bit index math, every offset computed before the select, so
          // the selects stay selects (a branch around the loads would make
          // the compiler wait for each load before the next)
          const uint32_t nch32 = (uint32_t)nch, m32 = (uint32_t)M, nblk32 = (uint32_t)nblk;
          const uint32_t xrow_bytes = (uint32_t)(2 * K), xrb32 = (uint32_t)xrb;
#pragma unroll
          for (int q = 0; q < kXq; ++q) {
            const uint32_t i = (uint32_t)(lane + 64 * q);
            const uint32_t pc = i & 15u, rest = i >> 4;
            const uint32_t tk = rest / nch32, cc = rest - tk * nch32;
            const uint32_t b = 16u * cc + 2u * (uint32_t)wave + (pc >> 3);
            const uint32_t col = 128u * b + 16u * (pc & 7u);
            const bool ok = tk < m32 && b < nblk32;
            const uint32_t src = tk * xrow_bytes + col, dst = tk * xrb32 + col;
            xv[q] = buffer_load16(xres, ok ? src : 0x80000000u);
            xdst[q] = ok ? dst : 0xFFFFFFFFu;
          }
        }
      } else {
        if (c < 2) load_xc(cl(c), X[c]);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (XL) {
      // the wave's own pieces and zero area; its later reads follow in order
#pragma unroll
      for (int q = 0; q < kXq; ++q)
        if (xdst[q] != 0xFFFFFFFFu) *reinterpret_cast<u32x4_t*>(xl + xdst[q]) = xv[q];
      if (lane < 8) *reinterpret_cast<u32x4_t*>(xl + M * xrb + 128 * wave + 16 * lane) = zero;
    }
    // chunk 0's DMA: followed by its scales, the x loads (XL: kXq, XD: none
    // -- x of chunk 0 went first -- else two chunks of 8) and kAhead - 1
    // DMA + scale pairs
    __builtin_amdgcn_s_waitcnt(
        waitcnt_imm(2 + (XL ? kXq : XD ? 0 : 16) + 4 * (kAhead - 1), 0));

    // x operand j of chunk ch from LDS: token lr's 16 bytes at k = 64 b + 8 j
    auto x_lds = [&](int64_t ch) {
      const int64_t b = blk_of(ch);
      const uint32_t xa = (tok_ok && b < nblk) ? (uint32_t)(lr * xrb + 128 * b)
                                                : (uint32_t)(M * xrb + 128 * wave);
      return [=](int j) -> u32x4_t {
        return *reinterpret_cast<const u32x4_t*>(xl + xa + 16 * j);
      };
    };

    // phase = ch mod NST: the stage read (rd), the stage filled (fill),
    // the scale set and the x set (ch mod 3) are then compile-time choices
    auto iteration = [&](int64_t ch, auto phase, auto wait, const u32x4_t* __restrict__ rd,
                         u32x4_t* __restrict__ fill, const uint8_t* __restrict__ xrd,
                         uint8_t* __restrict__ xfill) {
      constexpr int ph = decltype(phase)::value;
      constexpr int W = decltype(wait)::value;
      static_assert(XL || XD || NST % 3 == 0, "x sets rotate with the phase");
      if constexpr (XD) {
        dma_x(xfill, cl(ch + 1));
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!XL) {
        load_xc(cl(ch + 2), X[(ph + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
      dma_codes(fill, cl(ch + kAhead));
      load_scale(cl(ch + kAhead), Sc[(ph + kAhead) % NST]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (XD)
        decode_chunk(rd, ch, Sc[ph], x_ring(xrd));
      else if constexpr (XL)
        decode_chunk(rd, ch, Sc[ph], x_lds(ch));
      else
        decode_chunk(rd, ch, Sc[ph], [&](int j) -> u32x4_t { return X[ph % 3][j]; });
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(W, 0));
    };
    static_assert(6 % NST == 0, "the loop below is unrolled by six iterations");
    u32x4_t* const R[6] = {ring, ring + kStageU4, ring + 2 * kStageU4,
                           ring + 3 * kStageU4, ring + 4 * kStageU4, ring + 5 * kStageU4};
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using P4 = std::integral_constant<int, 4>;
    using P5 = std::integral_constant<int, 5>;
    // iteration ch (phase ch mod 6 here) reads stage ch mod NST and fills
    // stage ch + kAhead (mod NST), the one it read kAhead - NST iterations ago
    // (XD: x stage ch mod 2 is read, the other filled)
    auto step = [&](int64_t ch, auto phase6, auto wait) {
      constexpr int ph = decltype(phase6)::value % NST;
      constexpr int xs = decltype(phase6)::value % 2;
      iteration(ch, std::integral_constant<int, ph>(), wait, R[ph], R[(ph + kAhead) % NST],
                xdr + kXdStage * xs, xdr + kXdStage * (1 - xs));
    };
    using WS = std::integral_constant<int, kWaitSteady>;
    constexpr auto lo = [](int a, int b) { return a < b ? a : b; };
    constexpr int kWaitMin =
        lo(lo(lo(wait_for(0), wait_for(1)), lo(wait_for(2), wait_for(3))), lo(wait_for(4), kWaitSteady));
    using WM = std::integral_constant<int, kWaitMin>;
    if (nch >= 6) {
      step(0, P0(), std::integral_constant<int, wait_for(0)>());
      step(1, P1(), std::integral_constant<int, wait_for(1)>());
      step(2, P2(), std::integral_constant<int, wait_for(2)>());
      step(3, P3(), std::integral_constant<int, wait_for(3)>());
      step(4, P4(), std::integral_constant<int, wait_for(4)>());
      step(5, P5(), WS());
      int64_t ch = 6;
      for (; ch + 6 <= nch; ch += 6) {
        step(ch, P0(), WS());
        step(ch + 1, P1(), WS());
        step(ch + 2, P2(), WS());
        step(ch + 3, P3(), WS());
        step(ch + 4, P4(), WS());
        step(ch + 5, P5(), WS());
      }
      if (ch < nch) step(ch, P0(), WS());
      if (ch + 1 < nch) step(ch + 1, P1(), WS());
      if (ch + 2 < nch) step(ch + 2, P2(), WS());
      if (ch + 3 < nch) step(ch + 3, P3(), WS());
      if (ch + 4 < nch) step(ch + 4, P4(), WS());
    } else {
      step(0, P0(), WM());
      if (1 < nch) step(1, P1(), WM());
      if (2 < nch) step(2, P2(), WM());
      if (3 < nch) step(3, P3(), WM());
      if (4 < nch) step(4, P4(), WM());
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
      if (p.keep || p.rng) {
        // LoRA dropout on the adapter's input: piece j of the lane's token
        // row is mask byte (m, k / 8) with k = kb + 8 j (lanes past the M
        // tokens read token 0's row and bytes; their columns are never
        // stored)
        const uint32_t c0 = (uint32_t)((tok_ok ? lr : 0) * (K / 8) + (kb < K ? kb : 0) / 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t kbyte = p.rng ? philox_keep_byte(p.drop, c0 + (uint32_t)j)
                                       : (uint32_t)p.keep[c0 + j];
          xb[j] = keep8(xb[j], kbyte);
        }
      }
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
  // (token m, row) pairs of the tile: consecutive threads, consecutive rows
  constexpr int kPairs = 32 * kDecodeMaxM / (WAVES * 64);
  float sum[kPairs];
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int e = t + WAVES * 64 * i, m = e >> 5, row = e & 31;
    sum[i] = 0.0f;
    if (e < 32 * mcols) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) sum[i] += red[(w * 32 + row) * mcols + m];
    }
  }
  if (a_tile) {  // this split's partial of x . A^T, rows n0 .. n0 + 31 of A
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int e = t + WAVES * 64 * i, m = e >> 5, row = e & 31;
      if (e < 32 * mcols && n0 + row < nrows)
        p.part[((int64_t)z * M + m) * p.r + n0 + row] = sum[i];
    }
    return;
  }
  const int r = p.r;
  if (r == 0) {  // no adapter: the sums are y
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int e = t + WAVES * 64 * i, m = e >> 5, row = e & 31;
      if (e < 32 * mcols && n0 + row < N)
        p.y[(int64_t)m * N + n0 + row] = __builtin_bit_cast(uint16_t, (__bf16)sum[i]);
    }
    return;
  }
  // The adapter term: y = bf16(sum + scale . sum_j xa[m][j] B[n][j]), with
  // xa[m][j] = sum_z part[z][m][j] added in split order (the A tiles ran
  // before this launch).  xa [M][r] fp32 and the tile's 32 rows of B (bf16,
  // rows padded by 4 bytes against bank conflicts) replace the wave sums in
  // LDS; the r-sum runs in fp32 on the vector units (32 M r multiply-adds
  // per block).  Loads go through buffer descriptors, so splits past sa
  // and rows past N read zero and need no branch.
  __syncthreads();  // every thread has read its wave sums
  static_assert(kDecodeMaxM * 256 * 4 <= 32 * 1024, "xa [M][r] fits below B's rows");
  static_assert(32 * 1024 + 32 * (256 + 2) * 2 <= kTabBytes + ring_bytes(NSTAGE_XL),
                "B's rows fit in the smallest variant's LDS");
  float* xs = red;
  uint16_t* bs = reinterpret_cast<uint16_t*>(lds + 32 * 1024);
  const int brow = r + 2;
  const int64_t nxa = M * r;
  const __amdgpu_buffer_rsrc_t pres = make_rsrc(p.part, (uint32_t)(p.sa * nxa * 4));
  const __amdgpu_buffer_rsrc_t bres = make_rsrc(p.B, (uint32_t)(N * r * 2));
  constexpr int EPT = 2;
  for (int64_t e0 = t; e0 < nxa; e0 += WAVES * 64 * EPT) {
    float v[EPT][kMaxASplits];
#pragma unroll
    for (int u = 0; u < EPT; ++u)
#pragma unroll
      for (int zz = 0; zz < kMaxASplits; ++zz) {
        const int64_t e = e0 + WAVES * 64 * u;
        const uint32_t off = e < nxa ? (uint32_t)((zz * nxa + e) * 4) : 0x80000000u;
        v[u][zz] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pres, off, 0, 0));
      }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int64_t e = e0 + WAVES * 64 * u;
      float a = v[u][0];
#pragma unroll
      for (int zz = 1; zz < kMaxASplits; ++zz) a += v[u][zz];
      if (e < nxa) xs[e] = a;
    }
  }
  for (int e = t; e < 16 * r; e += WAVES * 64) {  // 32 rows x r bf16 as 2-element words
    const int row = e / (r / 2), jj = 2 * (e - row * (r / 2));
    const uint32_t off = (uint32_t)(((n0 + row) * r + jj) * 2);
    const uint32_t w2 = __builtin_amdgcn_raw_buffer_load_b32(bres, off, 0, 0);
    *reinterpret_cast<uint32_t*>(bs + row * brow + jj) = w2;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int e = t + WAVES * 64 * i, m = e >> 5, row = e & 31;
    if (e < 32 * mcols && n0 + row < N) {
      const float* xm = xs + m * r;
      const uint16_t* bn = bs + row * brow;
      float a = 0.0f;
      for (int j = 0; j < r; j += 2) {
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(bn + j);
        a = fmaf(xm[j], bf16_bits_to_f32(w2 & 0xFFFFu), a);
        a = fmaf(xm[j + 1], bf16_bits_to_f32(w2 >> 16), a);
      }
      p.y[(int64_t)m * N + n0 + row] =
          __builtin_bit_cast(uint16_t, (__bf16)(sum[i] + p.scale * a));
    }
  }
}

namespace {

// k splits of the adapter's A tiles, which run in a launch of their own
// before the weight tiles: pieces of about 512 k (at most 16, the planes the
// weight tiles' epilogue adds), so each takes about one memory round trip
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
  return M * (2 * K + 16) + WAVES * 128 <= kXBytes && M * nch * 16 <= 64 * kXq;
}

int decode_splits(int64_t M, int64_t N, int64_t K, int r) {
  (void)M;
  (void)N;
  return r > 0 ? a_splits(K) : 0;
}

hipError_t launch_decode_fwd(const uint8_t* codes, const uint8_t* qscale, const float* step,
                             const float* dq_mean, const uint16_t* x, const uint16_t* A,
                             const uint16_t* B, int r,
                             float scale, float* part, int splits, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, const Nf4Levels& L, hipStream_t s,
                             const uint8_t* keep, const PhiloxDrop* drop) {
  DecodeParams p;
  p.keep = keep;
  p.drop = drop ? *drop : PhiloxDrop{};
  p.rng = drop != nullptr;
  p.codes = codes;
  p.qscale = qscale;
  p.step = step;
  p.dq_mean = dq_mean;
  p.x = x;
  p.A = A;
  p.B = B;
  p.part = part;
  p.M = M;
  p.N = N;
  p.K = K;
  p.r = r;
  p.scale = scale;
  p.y = y;
  p.sa = r > 0 ? a_splits(K) : 1;
  if (r > 0 && (p.sa > splits || part == nullptr)) return hipErrorInvalidValue;
  p.L = L;
  const dim3 block(WAVES * 64);
  if (r > 0) {
    // the A tiles alone: x . A^T partials for the weight tiles' epilogue
    DecodeParams pa = p;
    pa.w_blocks = 0;
    pa.blocks = (int64_t)((r + 31) / 32) * p.sa;
    hipLaunchKernelGGL((decode_main_kernel<0, false>), dim3((unsigned)pa.blocks), block, 0, s,
                       pa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  p.w_blocks = (N + 31) / 32;
  p.blocks = p.w_blocks;
  const dim3 grid((unsigned)p.blocks);
  const int xm = decode_x_in_lds(M, K) ? 1 : (M <= kXdTok ? 2 : 0);
  if (dq_mean) {
    if (xm == 1)
      hipLaunchKernelGGL((decode_main_kernel<1, true>), grid, block, 0, s, p);
    else if (xm == 2)
      hipLaunchKernelGGL((decode_main_kernel<2, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((decode_main_kernel<0, true>), grid, block, 0, s, p);
  } else {
    if (xm == 1)
      hipLaunchKernelGGL((decode_main_kernel<1, false>), grid, block, 0, s, p);
    else if (xm == 2)
      hipLaunchKernelGGL((decode_main_kernel<2, false>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((decode_main_kernel<0, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace qlora
