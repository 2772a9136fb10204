// Adapter merge for export: W_m = W_base + s . B . A, s = alpha / r.
//
// [QLoRA -- the democratization event, deployment note]: the merged model
// is made by dequantising the base, merging the adapter in, and possibly
// quantising again.  [QLoRA / infivelines.com, the recipe's last step]:
// merging into the 4-bit base and saving loses precision twice; merge
// against the original weights.  [QLoRA, and fine-tuning a 7B model on a
// free GPU, "Merging a QLoRA adapter"]: merging into the full-precision base
// is the usual practice.  W_base is therefore either the decoded NF4 base
// (bit-identical to the dequantiser) or the original fp32 weight.
//
// The update B . A is a rank-r contraction, run on MFMA 32x32x16 bf16 with
// the roles chosen so that each lane ends up holding 4 consecutive columns
// of one output row:
//   a-operand  A^T: row i = column k of A, reduction index j (A is [r, K])
//   b-operand  B^T: column = row n of B, reduction index j (B is [N, r])
//   D[i = k][j = n]: lane l holds n = n0 + l % 32 and, in accumulator v,
//   k = k0 + 8 (v / 4) + 4 (l / 32) + v % 4.
// One wave owns a 64-column strip of k (two such 32-column MFMA tiles; for
// the NF4 base, one block of every row) and walks a range of 32-row tiles
// of n; its A fragments stay in registers for the whole walk.  Per tile it
// reads 32 rows of B (an L2-resident [N, r] array) and the base (32 bytes of
// codes per row, or fp32), and writes the tile as fp32 and/or bf16, staged
// through LDS so that every store covers whole 128-byte lines, which are
// then streamed out with nontemporal stores.  The path is bound
// by HBM traffic: about 0.52 (NF4) or 4 (fp32) bytes read and 4 + 2 bytes
// written per weight.
//
// fp32 result: fl32(W_base + s . U) with one rounding (fma), U the MFMA's
// fp32 sum of the exact bf16 products; bf16 result: that fp32 value rounded
// to nearest even.

#include "launch.h"

namespace qlora {
namespace {

constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every tensor: loads return 0

struct MergeArgs {
  const uint8_t* codes;   // NF4 base (or null)
  const uint8_t* qscale;
  const float* step;
  const float* dq_mean;   // the mean-centred scale format's mean (or null)
  const float* w0;        // fp32 original base (or null)
  const uint16_t* A;      // [r, K] bf16
  const uint16_t* B;      // [N, r] bf16 (never null: any readable pointer when r = 0)
  float* out_f32;         // [N, K] or null
  uint16_t* out_bf16;     // [N, K] or null
  int64_t N, K;
  int r;
  float scale;
  int strips;             // K / 64
  int tiles_per_wave;     // 32-row tiles of n per wave
  int waves;              // strips * ceil((N / 32) / tiles_per_wave)
};

__device__ __forceinline__ float lo_bf16(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t pair) {
  return __uint_as_float(pair & 0xFFFF0000u);
}

constexpr int kSlabF = 64 + 4;                // fp32 staging row: 64 values + 16 B pad
constexpr int kSlabFloats = 32 * kSlabF;      // per wave

// One tile's inputs, loaded ahead of its use.
template <int RS, bool NF4>
struct TileIn {
  u32x4_t b[RS];                // B fragments (shared by the strip's two halves)
  u32x4_t base[NF4 ? 2 : 8];    // the row's 64 codes (NF4) or this lane's 32 fp32
  uint32_t q;                   // NF4: 8-bit block scale of the row's block
  float st;                     // NF4: its group step
};

template <int RS, bool NF4>
__device__ __forceinline__ void load_tile(const MergeArgs& a, __amdgpu_buffer_rsrc_t rb,
                                          int64_t n0, int64_t k0, int c, int h,
                                          TileIn<RS, NF4>& t) {
  const int64_t n = n0 + c;
  const uint32_t brow = (uint32_t)(n * a.r) * 2u;
#pragma unroll
  for (int js = 0; js < RS; ++js) {
    const int j = 16 * js + 8 * h;
    const uint32_t off = j < a.r ? brow + 2u * (uint32_t)j : kOob;
    t.b[js] = buffer_load16(rb, off);
  }
  const int64_t e = n * a.K + k0;  // flattened index of the row's first strip element
  if constexpr (NF4) {
    // the strip is one whole 64-weight block of the row
    const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(a.codes + (e >> 1));
    t.base[0] = cp[0];
    t.base[1] = cp[1];
    const int64_t blk = e >> 6;
    t.q = a.qscale[blk];
    t.st = a.step[blk >> 8];
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        t.base[4 * s + g] =
            *reinterpret_cast<const u32x4_t*>(a.w0 + e + 32 * s + 8 * g + 4 * h);
  }
}

// One tile: W_m rows t*32 .. t*32+31 of the wave's 64-column strip, from
// inputs loaded earlier.  The fp32 results leave the MFMA layout (one row
// per lane pair) through the wave's LDS slab and come back row-major, so
// that every store instruction writes whole rows of the strip: 4 rows x
// 256 B (fp32) or 4 rows x 128 B (bf16, rounded from the same values).
// OUT bit 0: fp32 output, bit 1: bf16 output.
template <int RS, bool NF4, int OUT>
__device__ __forceinline__ void merge_tile(const MergeArgs& a, const Nf4Levels& L,
                                           const u32x4_t (&af)[2][RS],
                                           const TileIn<RS, NF4>& in, float* slab, int64_t t,
                                           int64_t k0, int lane) {
  const int c = lane & 31, h = lane >> 5;
  Nf4Lut lut;
  if constexpr (NF4) lut = nf4_make_lut(L, nf4_block_scale(in.q, in.st, scale_fmt(a.dq_mean)));
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // zero-padded reduction steps (j >= r) multiply zeros: no guard needed
    f32x16_t acc = {};
#pragma unroll
    for (int js = 0; js < RS; ++js) acc = mfma32x32x16(af[s][js], in.b[js], acc);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float w[4];
      if constexpr (NF4) {
        // this lane's 4 codes: bytes 16s + 4g + 2h, +1 of the row's 32
        const uint32_t word = in.base[s][g];
        const uint32_t v16 = h ? word >> 16 : word & 0xFFFFu;
        const uint32_t ev = v16 & 0x0F0Fu, od = (v16 >> 4) & 0x0F0Fu;
        uint32_t o01, o23;
        nf4_lookup4(lut, perm(od, ev, 0x05010400u), o01, o23);
        w[0] = lo_bf16(o01); w[1] = hi_bf16(o01);
        w[2] = lo_bf16(o23); w[3] = hi_bf16(o23);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(in.base[4 * s + g][i]);
      }
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(a.scale, acc[4 * g + i], w[i]);
      *reinterpret_cast<f32x4_t*>(slab + c * kSlabF + 32 * s + 8 * g + 4 * h) = v;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int rr = lane >> 4, cc = 4 * (lane & 15);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(slab + (4 * p + rr) * kSlabF + cc);
    const int64_t off = (t * 32 + 4 * p + rr) * a.K + k0 + cc;
    // whole lines, written once and not read back here: streamed past the
    // caches (nontemporal) rather than allocated in L2
    if constexpr (OUT & 1)
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(a.out_f32 + off));
    if constexpr (OUT & 2) {
      const u32x2_t b = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      __builtin_nontemporal_store(b, reinterpret_cast<u32x2_t*>(a.out_bf16 + off));
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int RS, bool NF4, int OUT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, Nf4Levels L) {
  __shared__ float slabs[4 * kSlabFloats];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = (int)blockIdx.x * 4 + wave;
  if (gw >= a.waves) return;
  float* slab = slabs + wave * kSlabFloats;
  const int strip = gw % a.strips;
  const int64_t chunk = gw / a.strips;
  const int64_t k0 = (int64_t)strip * 64;
  const int64_t n_tiles = a.N >> 5;
  const int64_t t0 = chunk * a.tiles_per_wave;
  const int64_t t1 = t0 + a.tiles_per_wave < n_tiles ? t0 + a.tiles_per_wave : n_tiles;
  const int c = lane & 31, h = lane >> 5;

  // A^T fragments of the two 32-column halves: lane (c, h) holds
  // A[16 js + 8 h + 0..7][k0 + 32 s + c]
  u32x4_t af[2][RS];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int js = 0; js < RS; ++js) {
      const int j = 16 * js + 8 * h;
      u32x4_t f = {0u, 0u, 0u, 0u};
      if (j < a.r) {
        const uint16_t* p = a.A + (int64_t)j * a.K + k0 + 32 * s + c;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          f[t] = (uint32_t)p[(2 * t) * a.K] | ((uint32_t)p[(2 * t + 1) * a.K] << 16);
      }
      af[s][js] = f;
    }

  // Two tiles in flight, ping-pong: each tile's successor is loaded before
  // its stores are issued (past the end, the last tile is loaded again
  // rather than branching around the loads).
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B, (uint32_t)(a.N * a.r * 2));
  const int64_t last = t1 - 1;
  TileIn<RS, NF4> p0, p1;
  load_tile<RS, NF4>(a, rb, t0 * 32, k0, c, h, p0);
  for (int64_t t = t0; t < t1; t += 2) {
    load_tile<RS, NF4>(a, rb, (t + 1 < last ? t + 1 : last) * 32, k0, c, h, p1);
    merge_tile<RS, NF4, OUT>(a, L, af, p0, slab, t, k0, lane);
    if (t + 1 >= t1) break;
    load_tile<RS, NF4>(a, rb, (t + 2 < last ? t + 2 : last) * 32, k0, c, h, p0);
    merge_tile<RS, NF4, OUT>(a, L, af, p1, slab, t + 1, k0, lane);
  }
}

template <int RS, bool NF4>
hipError_t launch_out(int out, const MergeArgs& a, const Nf4Levels& L, int grid,
                      hipStream_t s) {
  if (out == 1)
    hipLaunchKernelGGL((merge_kernel<RS, NF4, 1>), dim3(grid), dim3(256), 0, s, a, L);
  else if (out == 2)
    hipLaunchKernelGGL((merge_kernel<RS, NF4, 2>), dim3(grid), dim3(256), 0, s, a, L);
  else
    hipLaunchKernelGGL((merge_kernel<RS, NF4, 3>), dim3(grid), dim3(256), 0, s, a, L);
  return hipGetLastError();
}

template <int RS>
hipError_t launch_rs(bool nf4, int out, const MergeArgs& a, const Nf4Levels& L, int grid,
                     hipStream_t s) {
  return nf4 ? launch_out<RS, true>(out, a, L, grid, s)
             : launch_out<RS, false>(out, a, L, grid, s);
}

}  // namespace

MergePlan merge_plan(int64_t N, int64_t K) {
  MergePlan p;
  const int64_t strips = K / 64, n_tiles = N / 32;
  const int64_t total = strips * n_tiles;
  int64_t tpw = (total + kMergeTargetWaves - 1) / kMergeTargetWaves;
  if (tpw < 1) tpw = 1;
  if (tpw > n_tiles) tpw = n_tiles;
  p.tiles_per_wave = (int)tpw;
  p.waves = strips * ((n_tiles + tpw - 1) / tpw);
  p.blocks = (p.waves + 3) / 4;
  return p;
}

hipError_t launch_merge(const uint8_t* codes, const uint8_t* qscale, const float* step,
                        const float* dq_mean, const float* w0, const uint16_t* A,
                        const uint16_t* B, int r,
                        float scale, float* out_f32, uint16_t* out_bf16, int64_t N, int64_t K,
                        const Nf4Levels& L, hipStream_t s) {
  const MergePlan p = merge_plan(N, K);
  MergeArgs a;
  a.codes = codes;
  a.qscale = qscale;
  a.step = step;
  a.dq_mean = dq_mean;
  a.w0 = w0;
  a.A = A;
  a.B = r > 0 ? B : reinterpret_cast<const uint16_t*>(codes ? (const void*)codes : (const void*)w0);
  a.out_f32 = out_f32;
  a.out_bf16 = out_bf16;
  a.N = N;
  a.K = K;
  a.r = r;
  a.scale = scale;
  a.strips = (int)(K / 64);
  a.tiles_per_wave = p.tiles_per_wave;
  a.waves = (int)p.waves;
  const bool nf4 = codes != nullptr;
  const int out = (out_f32 ? 1 : 0) | (out_bf16 ? 2 : 0);
  const int grid = (int)p.blocks;
  if (r <= 16) return launch_rs<1>(nf4, out, a, L, grid, s);
  if (r <= 32) return launch_rs<2>(nf4, out, a, L, grid, s);
  if (r <= 64) return launch_rs<4>(nf4, out, a, L, grid, s);
  if (r <= 128) return launch_rs<8>(nf4, out, a, L, grid, s);
  return launch_rs<16>(nf4, out, a, L, grid, s);
}

}  // namespace qlora
