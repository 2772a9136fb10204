// Device helpers shared by the gfx950 kernels: vector types, bf16 packing,
// byte permutes, and the NF4 decode (a per-block 16-entry bf16 table looked
// up with v_perm_b32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Compute-type traits (bf16 or fp16), defined with the MFMA wrappers below.
struct Bf16T;
struct F16T;

// The 16 fp32 NF4 levels, passed to kernels by value (lands in SGPRs).
struct Nf4Levels {
  float v[16];
};
struct Nf4Thresholds {
  float t[15];
};

// Code lookup for the quantiser.  bin(u) = min(63, trunc(32 * fl32(u + 1)))
// is monotone in u, so for |u| <= 1 the code #{i : u > t[i]} equals
// base[bin] + (u > thr[bin]), where base[b] counts the thresholds whose bin
// is below b and thr[b] is the threshold inside bin b (+2, above every u,
// if there is none; no bin holds two).
struct Nf4CodeBins {
  float thr[64];
  uint32_t base[64];
};
__host__ __device__ __forceinline__ uint32_t nf4_bin(float u) {
  const float t = (u + 1.0f) * 32.0f;  // the product is exact (power of two)
  const uint32_t b = (uint32_t)t;
  return b < 63u ? b : 63u;
}

// v_perm_b32: result byte i = byte sel.byte[i] of the 8-byte value
// {hi:lo}; selector 0..3 picks lo's bytes, 4..7 hi's bytes, 12 gives 0x00
// and 13..15 give 0xFF.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// ---------------------------------------------------------------------------
// NF4 decode.  A block's 16 decoded values e[c] = bf16_rne(fp32(L[c] * s'))
// are held as two 16-byte planes: lo[j] holds the low bytes of entries
// 4j..4j+3, hi[j] their high bytes.  One v_perm picks 4 bytes out of 8, so
// a 4-bit code is resolved with one perm into entries 0..7, one into 8..15,
// and a third perm that keeps the right one (chosen by the code's bit 3).
// ---------------------------------------------------------------------------
struct Nf4Lut {
  uint32_t lo[4];
  uint32_t hi[4];
};

template <class DT = Bf16T>
__device__ __forceinline__ Nf4Lut nf4_make_lut(const Nf4Levels& L, float scale) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // one fp32 product per level, then round-to-nearest-even to the
    // compute type
    const float a = L.v[2 * i] * scale;
    const float b = L.v[2 * i + 1] * scale;
    p[i] = DT::pack2(a, b);
  }
  Nf4Lut t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.lo[j] = perm(p[2 * j + 1], p[2 * j], 0x06040200u);
    t.hi[j] = perm(p[2 * j + 1], p[2 * j], 0x07050301u);
  }
  return t;
}

// 4 codes, one per byte (values 0..15) -> two bf16 pairs, in byte order.
__device__ __forceinline__ void nf4_lookup4(const Nf4Lut& t, uint32_t n,
                                            uint32_t& o01, uint32_t& o23) {
  const uint32_t n_hi = n & 0x07070707u;                          // index in 8..15
  const uint32_t pick = ((n >> 1) & 0x04040404u) | 0x03020100u;   // j or j+4
  const uint32_t lo = perm(perm(t.lo[3], t.lo[2], n_hi), perm(t.lo[1], t.lo[0], n), pick);
  const uint32_t hi = perm(perm(t.hi[3], t.hi[2], n_hi), perm(t.hi[1], t.hi[0], n), pick);
  o01 = perm(hi, lo, 0x05010400u);
  o23 = perm(hi, lo, 0x07030602u);
}

// 8 packed codes (byte j = c[2j] | c[2j+1] << 4) -> 8 bf16 in element order
// as four pairs: out[i] = e[c(2i)] | e[c(2i+1)] << 16.
__device__ __forceinline__ u32x4_t nf4_decode8(const Nf4Lut& t, uint32_t v) {
  const uint32_t ev = v & 0x0F0F0F0Fu;          // c0 c2 c4 c6
  const uint32_t od = (v >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
  const uint32_t n0 = perm(od, ev, 0x05010400u);  // c0 c1 c2 c3
  const uint32_t n1 = perm(od, ev, 0x07030602u);  // c4 c5 c6 c7
  uint32_t o0, o1, o2, o3;
  nf4_lookup4(t, n0, o0, o1);
  nf4_lookup4(t, n1, o2, o3);
  const u32x4_t out = {o0, o1, o2, o3};
  return out;
}

// The block-scale format of a weight.  Unsigned (the default): the byte q
// is 0..255 and s' = fp32(q * step).  Mean-centred (the paper-style
// variant): the byte is a two's-complement code and s' =
// fp32(fp32(q * step) + mean).  One formula serves both: the signed value
// is (q ^ sx) - sx with sx = 0x80 (centred) or 0 (unsigned), and the
// unsigned format adds mu = +0, which leaves its non-negative product
// unchanged.
struct ScaleFmt {
  uint32_t sx;
  float mu;
};
__device__ __forceinline__ ScaleFmt scale_fmt(const float* dq_mean) {
  ScaleFmt f;
  f.sx = dq_mean ? 0x80u : 0u;
  f.mu = dq_mean ? *dq_mean : 0.0f;
  return f;
}

// Decoded block scale of the unsigned format: s' = fp32(q * step) (q
// converts exactly; one rounding).
__device__ __forceinline__ float nf4_block_scale(uint32_t q, float step) {
  return static_cast<float>(q) * step;
}

// Decoded block scale of either format: the code converts exactly, and the
// product and the sum are each rounded once (never fused).
__device__ __forceinline__ float nf4_block_scale(uint32_t q, float step, ScaleFmt f) {
#pragma clang fp contract(off)
  const float prod = static_cast<float>((int)(q ^ f.sx) - (int)f.sx) * step;
  return prod + f.mu;
}

// ---------------------------------------------------------------------------
// Counter-based draws for LoRA dropout: Philox4x32 with ten rounds (Salmon,
// Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC 2011).  A round forms the 64-bit products M0 * X0 and M1 * X2 and maps
// (X0, X1, X2, X3) to (hi1 ^ X1 ^ K0, lo1, hi0 ^ X3 ^ K1, lo0); the key
// advances by the Weyl constants between rounds.
//
// The keep bits of one 8-element chunk of an activation come from one call:
// counter (chunk index, 0, offset lo, offset hi) -- the chunk index is the
// byte of the packed [M, K/8] mask, below 2^32 for every tensor the library
// accepts -- and key (seed lo, seed hi).  Element j takes the 16-bit half
// j % 2 (low first) of word j / 2 and is kept iff it is >= t.
// ---------------------------------------------------------------------------
struct PhiloxDrop {
  uint32_t k0, k1;    // key: the seed
  uint32_t o0, o1;    // counter words 2, 3: the stream offset
  uint32_t t;         // threshold: nearest integer to 65536 p
};

__device__ __forceinline__ u32x4_t philox4x32_10(u32x4_t x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x[2];
    x = u32x4_t{(uint32_t)(p1 >> 32) ^ x[1] ^ k0, (uint32_t)p1,
                (uint32_t)(p0 >> 32) ^ x[3] ^ k1, (uint32_t)p0};
  }
  return x;
}

// LoRA dropout: the 8 bf16 of a 16-byte chunk (consecutive k, value i in
// halfword i) keep their bits where bit i of the chunk's keep byte is set
// and become +0 where it is clear.
__device__ __forceinline__ u32x4_t keep8(const u32x4_t v, uint32_t kb) {
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t b = kb >> (2 * d);
    o[d] = v[d] & (((b & 1u) ? 0x0000FFFFu : 0u) | ((b & 2u) ? 0xFFFF0000u : 0u));
  }
  return o;
}

// The keep byte of mask byte `chunk` (bit j set where element 8 chunk + j
// of the flattened [M, K] activation is kept).
__device__ __forceinline__ uint32_t philox_keep_byte(const PhiloxDrop& d, uint32_t chunk) {
  const u32x4_t w = philox4x32_10(u32x4_t{chunk, 0u, d.o0, d.o1}, d.k0, d.k1);
  uint32_t kb = 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    kb |= ((w[h] & 0xFFFFu) >= d.t ? 1u : 0u) << (2 * h);
    kb |= ((w[h] >> 16) >= d.t ? 1u : 0u) << (2 * h + 1);
  }
  return kb;
}

// Raw buffer access (gfx9 descriptor: untyped dwords, DATA_FORMAT 32).
// Loads at byte offsets at or past `bytes` return zero, which the GEMMs use
// for rows beyond the tensor instead of branching.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same with a wave-uniform part of the offset in the scalar operand
// (soff must be uniform).  The range check covers the lane offset only, so
// soff may not carry a term that is meant to push a lane out of range.
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buffer_load1(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Block-to-tile mapping for a 1-D grid of `total` blocks.  Consecutive
// workgroup ids are dealt round-robin to the 8 XCDs (each with its own L2),
// so id i is first turned into a rank that is contiguous within its XCD;
// ranks are then walked in groups of `group_m` row tiles (column tiles
// fastest within a group), so the blocks resident on one XCD share a few
// activation tiles and a few weight tiles at every k step.
struct TileCoord {
  int64_t m, n, z;
};
// tile rank (0 .. m_tiles * n_tiles - 1) -> (m, n) in the grouped order
__device__ __forceinline__ void tile_of_rank(int64_t tr, int64_t m_tiles, int64_t n_tiles,
                                             int group_m, int64_t& m, int64_t& n) {
  const int64_t span = (int64_t)group_m * n_tiles;
  const int64_t g = tr / span, w = tr - g * span;
  const int64_t gm = (m_tiles - g * group_m) < group_m ? (m_tiles - g * group_m) : group_m;
  m = g * group_m + w % gm;
  n = w / gm;
}
__device__ __forceinline__ TileCoord xcd_tile(int64_t id, int64_t total, int64_t m_tiles,
                                              int64_t n_tiles, int group_m) {
  constexpr int kXcd = 8;
  const int64_t xcd = id % kXcd, slot = id / kXcd;
  const int64_t per = total / kXcd, extra = total % kXcd;
  const int64_t rank = xcd * per + (xcd < extra ? xcd : extra) + slot;
  const int64_t tiles = m_tiles * n_tiles;
  TileCoord c;
  c.z = rank / tiles;
  tile_of_rank(rank - c.z * tiles, m_tiles, n_tiles, group_m, c.m, c.n);
  return c;
}

// Work of one block of a fused GEMM grid.  Two schedules:
//  - uniform split (tail_q == 0): every tile's reduction is split over
//    `splits` blocks (1: none); block -> (tile, split z) by xcd_tile;
//  - split tail (tail_q > 0): the first `full` blocks each own one whole
//    tile (tile ranks 0 .. full-1); the last tail_q tiles, which would
//    otherwise run as a partly filled last round, are split tail_s ways
//    over the blocks after them, which write tile-local fp32 partials.
struct BlockWork {
  int64_t m, n;   // tile coordinates
  int z, nz;      // split index and count of this block's tile
  int64_t tail;   // tail tile index, or -1
};
__device__ __forceinline__ BlockWork block_work(int64_t id, int64_t total, int64_t m_tiles,
                                                int64_t n_tiles, int splits, int64_t full,
                                                int tail_q, int tail_s) {
  BlockWork w;
  if (tail_q == 0) {
    const TileCoord c = xcd_tile(id, total, m_tiles, n_tiles, 4);
    w.m = c.m;
    w.n = c.n;
    w.z = (int)c.z;
    w.nz = splits;
    w.tail = -1;
  } else if (id < full) {
    const TileCoord c = xcd_tile(id, full, m_tiles, n_tiles, 4);
    w.m = c.m;
    w.n = c.n;
    w.z = 0;
    w.nz = 1;
    w.tail = -1;
  } else {
    const int64_t e = id - full;
    w.tail = e % tail_q;
    w.z = (int)(e / tail_q);
    w.nz = tail_s;
    tile_of_rank(full + w.tail, m_tiles, n_tiles, 4, w.m, w.n);
  }
  return w;
}

// Epilogue of the fused GEMMs.  A wave holds a 32 NI (rows: n or k) x 32 NJ
// (columns: tokens m) fp32 tile as NI x NJ MFMA 32x32 tiles; lane l holds
// column 32 j + l % 32 and rows 32 i + 8 (v / 4) + 4 (l / 32) + v % 4.  The
// output is token-major (out[m][row]), so storing straight from registers
// would give every store instruction 32 rows of 16 bytes.  Instead each
// 32-column slice goes through the wave's own LDS area (32 x (32 NI + 4)
// fp32; the 4-float pad puts consecutive columns 4 banks apart) and comes
// back row-contiguous: 8 NI lanes then store one column's 32 NI rows.
// `part` selects fp32 partials, otherwise values are rounded to the
// compute type DT.
template <int NI>
constexpr int epi_stride() { return 32 * NI + 4; }
template <int NI>
constexpr int epi_floats() { return 32 * epi_stride<NI>(); }  // per wave
template <int NI, int NJ, class DT = Bf16T>
__device__ __forceinline__ void store_acc_tile(const f32x16_t (&acc)[NI][NJ], float* scratch,
                                               int64_t row0, int64_t col0, int64_t nrows,
                                               int64_t ncols, bool part, float* outf,
                                               uint16_t* outh, int64_t ld, int lane) {
  constexpr int S = epi_stride<NI>();
  constexpr int LPC = 8 * NI;      // lanes per column
  constexpr int CPP = 64 / LPC;    // columns per pass
  const int lr = lane & 31, lg = lane >> 5;
  const int rr = lane % LPC, cc = lane / LPC;
  const int64_t row = row0 + 4 * rr;  // the 4 rows this lane stores
  const bool row_ok = row < nrows;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]};
        *reinterpret_cast<f32x4_t*>(scratch + lr * S + 32 * i + 8 * q + 4 * lg) = v;
      }
#pragma unroll
    for (int pp = 0; pp < 32 / CPP; ++pp) {
      const int c = CPP * pp + cc;  // column within the slice
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(scratch + c * S + 4 * rr);
      const int64_t m = col0 + 32 * j + c;
      if (m < ncols && row_ok) {
        if (part) {
          *reinterpret_cast<f32x4_t*>(outf + m * ld + row) = v;
        } else {
          u32x2_t o;
          o[0] = DT::pack2(v[0], v[1]);
          o[1] = DT::pack2(v[2], v[3]);
          *reinterpret_cast<u32x2_t*>(outh + m * ld + row) = o;
        }
      }
    }
  }
}

// MFMA wrappers (gfx950 bf16, fp32 accumulate).
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The 16-bit compute type of a kernel: bf16 (the layer's) or fp16 (its
// fp16 compute-type variant).  Operands travel as raw 16-bit patterns;
// these are the only places the format matters: fp32 -> 16-bit conversion
// (round to nearest even), the MFMAs and the two-term dot product.
// (By-value helpers: a bit_cast of one element of a register vector to a
// 2-vector read element 0 whatever the index.)
struct Bf16T {
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ uint16_t cvt(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  static __device__ __forceinline__ float tof(uint16_t h) { return bf16_bits_to_f32(h); }
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return mfma32x32x16(a, b, c);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return mfma16x16x32(a, b, c);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
};
struct F16T {
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ uint16_t cvt(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
  static __device__ __forceinline__ float tof(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
  }
  static __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                  __builtin_bit_cast(f16x2_t, b), c, false);
  }
};

}  // namespace qlora
