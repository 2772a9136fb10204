// NF4 blockwise quantiser, 8-bit double quantisation of the block scales,
// and the standalone dequantiser (gfx950).
//
// [QLoRA / infivelines.com]: 16 NF4 levels at normal quantiles; one scale
// per block of 64 weights; the block scales quantised again in blocks of
// 256.  [QLoRA -- Module 12.4, "Design Details That Matter"]: NF4 and double
// quant.  The arithmetic of every step is fixed so that results are
// reproducible bit for bit: IEEE correctly rounded fp32 division, a
// round-half-even rint, one fp32 product per decoded value and a
// round-to-nearest-even bf16 conversion.  These kernels are HBM-bound
// streaming passes: every lane owns whole contiguous pieces so that loads
// and stores are wide and coalesced.

#include "device_common.h"
#include "launch.h"

namespace qlora {

// ---------------------------------------------------------------------------
// Quantiser: each lane owns 8 consecutive weights (two 16-byte loads), so 8
// lanes cover one 64-weight block and a wave covers 8 blocks.  The block's
// absmax m is a max over the 8 lanes (xor shuffles inside the 8-lane group).
//
// u = fl32(w / m) is formed without a division per weight: with
// y = fl32(1 / m), q = fl32(w * y) is within one ulp of w / m, the residual
// w - q * m is exact in one fma, and fl32(q + residual * y) is the correctly
// rounded quotient (Markstein's correction step; it needs no underflow, so
// blocks with m outside [2^-60, 2^60] divide directly).  The code is then
// base[bin(u)] + (u > thr[bin(u)]) from a 64-entry table in LDS: one
// comparison per weight instead of fifteen.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nf4_quantize_kernel(
    const float* __restrict__ w, int64_t n, uint8_t* __restrict__ codes,
    float* __restrict__ absmax, Nf4CodeBins bins) {
#pragma clang fp contract(off)
  __shared__ uint2 tab[64];
  if (threadIdx.x < 64)
    tab[threadIdx.x] = make_uint2(__float_as_uint(bins.thr[threadIdx.x]), bins.base[threadIdx.x]);
  __syncthreads();

  const int64_t lanes_total = (n + 7) >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
       g - (threadIdx.x & 7) < lanes_total;  // whole 8-lane groups iterate together
       g += stride) {
    const int64_t e0 = g << 3;
    float v[8];
    if (e0 + 8 <= n) {
      const float4* p = reinterpret_cast<const float4*>(w + e0);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? w[e0 + i] : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));

    float u[8];
    if (m >= 0x1p-60f && m <= 0x1p60f) {
      const float y = __fdiv_rn(1.0f, m);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = v[i] * y;
        const float res = __builtin_fmaf(-q, m, v[i]);  // exact
        u[i] = __builtin_fmaf(res, y, q);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = __fdiv_rn(v[i], m);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint2 t = tab[nf4_bin(u[i])];
      uint32_t c = t.y + (u[i] > __uint_as_float(t.x) ? 1u : 0u);
      if (!(m > 0.0f) || e0 + i >= n) c = 7;  // zero block, padding
      packed |= c << (4 * i);
    }
    if (e0 < n) {
      if (e0 + 8 <= n) {
        *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = packed;
      } else {
        const int64_t nbytes = (n + 1) >> 1;
        for (int i = 0; i < 4; ++i)
          if ((e0 >> 1) + i < nbytes) codes[(e0 >> 1) + i] = (uint8_t)(packed >> (8 * i));
      }
      if ((threadIdx.x & 7) == 0) absmax[e0 >> 6] = m;
    }
  }
}

// ---------------------------------------------------------------------------
// Quantiser and double quantisation in one pass: a workgroup of 1024 lanes
// owns one group of 256 blocks (16384 weights), each lane 16 consecutive
// weights (four 16-byte loads), four lanes per block.  The block absmax is
// a max over the 4 lanes, the lane's codes follow at once (they need only
// the block's absmax), and the group's step -- a max over the workgroup --
// comes last; every step uses exactly the arithmetic of
// nf4_quantize_kernel and double_quant_kernel, so the outputs are the same
// bits.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void nf4_quantize_dq_kernel(
    const float* __restrict__ w, int64_t n, uint8_t* __restrict__ codes,
    float* __restrict__ absmax, uint8_t* __restrict__ qscale, float* __restrict__ step_out,
    Nf4CodeBins bins) {
#pragma clang fp contract(off)
  __shared__ uint2 tab[64];
  __shared__ float wmax[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t < 64)
    tab[t] = make_uint2(__float_as_uint(bins.thr[t]), bins.base[t]);

  const int64_t g = blockIdx.x;
  const int64_t nb = (n + 63) >> 6;
  const int64_t e0 = g * 16384 + (int64_t)t * 16;  // this lane's 16 weights
  const int64_t b = e0 >> 6;                       // its block
  const bool full = e0 + 16 <= n;
  float v[16];
  if (full) {
    const float4* p = reinterpret_cast<const float4*>(w + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = p[i];
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (e0 + i < n) ? w[e0 + i] : 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));  // the block's absmax (0 past the end)
  __syncthreads();                    // the code table is in LDS

  // codes, as in nf4_quantize_kernel
  uint32_t packed[2] = {0u, 0u};
  const bool direct = m >= 0x1p-60f && m <= 0x1p60f;
  const float y = direct ? __fdiv_rn(1.0f, m) : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float u;
    if (direct) {
      const float q = v[i] * y;
      const float res = __builtin_fmaf(-q, m, v[i]);  // exact
      u = __builtin_fmaf(res, y, q);
    } else {
      u = __fdiv_rn(v[i], m);
    }
    const uint2 tt = tab[nf4_bin(u)];
    const uint32_t c = tt.y + (u > __uint_as_float(tt.x) ? 1u : 0u);
    packed[i >> 3] |= c << (4 * (i & 7));
  }
  if (!(m > 0.0f)) {  // zero block
    packed[0] = packed[1] = 0x77777777u;
  } else if (!full) {  // padding past n
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (e0 + i >= n)
        packed[i >> 3] = (packed[i >> 3] & ~(15u << (4 * (i & 7)))) | (7u << (4 * (i & 7)));
  }
  if (full) {
    const u32x2_t o = {packed[0], packed[1]};
    *reinterpret_cast<u32x2_t*>(codes + (e0 >> 1)) = o;
  } else if (e0 < n) {
    const int64_t nbytes = (n + 1) >> 1;
    for (int i = 0; i < 8; ++i)
      if ((e0 >> 1) + i < nbytes) codes[(e0 >> 1) + i] = (uint8_t)(packed[i >> 2] >> (8 * (i & 3)));
  }

  // the group's max over its 256 block scales (blocks past the end count 0)
  float gm = m;
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) gm = fmaxf(gm, __shfl_xor(gm, o, 64));
  if (lane == 0) wmax[wave] = gm;
  __syncthreads();
  gm = wmax[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) gm = fmaxf(gm, wmax[i]);
  const float st = __fdiv_rn(gm, 255.0f);
  if ((t & 3) == 0 && b < nb) {
    uint32_t q = 0;
    if (st > 0.0f) q = (uint32_t)fminf(rintf(__fdiv_rn(m, st)), 255.0f);
    qscale[b] = (uint8_t)q;
    absmax[b] = m;
  }
  if (t == 0) step_out[g] = st;
}

// ---------------------------------------------------------------------------
// Double quantisation: one wave per group of 256 scales, 4 scales per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void double_quant_kernel(
    const float* __restrict__ absmax, int64_t nb, uint8_t* __restrict__ qscale,
    float* __restrict__ step_out) {
  const int lane = threadIdx.x & 63;
  const int64_t groups = (nb + 255) >> 8;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t gidx = wave0; gidx < groups; gidx += wstride) {
    const int64_t b0 = (gidx << 8) + 4 * lane;
    float s[4];
    if (b0 + 4 <= nb) {
      const float4 a = *reinterpret_cast<const float4*>(absmax + b0);
      s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = (b0 + i < nb) ? absmax[b0 + i] : 0.0f;
    }
    float m = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float st = __fdiv_rn(m, 255.0f);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t q = 0;
      if (st > 0.0f) q = (uint32_t)fminf(rintf(__fdiv_rn(s[i], st)), 255.0f);
      packed |= q << (8 * i);
    }
    if (b0 + 4 <= nb) {
      *reinterpret_cast<uint32_t*>(qscale + b0) = packed;
    } else {
      for (int i = 0; i < 4; ++i)
        if (b0 + i < nb) qscale[b0 + i] = (uint8_t)(packed >> (8 * i));
    }
    if (lane == 0) step_out[gidx] = st;
  }
}

static int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

// ---------------------------------------------------------------------------
// Mean-centred double quantisation (the paper-style scale format).  The mean
// of all block scales is an fp64 sum in a fixed order -- each group's
// scales in index order, the group sums in kDqcChunks contiguous chunks,
// the chunk sums in chunk order -- so that it is reproducible bit for bit;
// then each group codes d = fp32(s - mean) on the symmetric grid
// step = fp32(max |d| / 127), q = clamp(rint(fp32(d / step)), -127, 127).
// ---------------------------------------------------------------------------
constexpr int kDqcChunks = 1024;

// one lane per group: its scales summed in index order (fp64)
__global__ __launch_bounds__(256) void dqc_group_sum_kernel(const float* __restrict__ absmax,
                                                            int64_t nb,
                                                            double* __restrict__ gsum) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t groups = (nb + 255) >> 8;
  if (g >= groups) return;
  const int64_t b0 = g << 8, b1 = b0 + 256 < nb ? b0 + 256 : nb;
  double acc = 0.0;
  int64_t b = b0;
  for (; b + 4 <= b1; b += 4) {
    const float4 v = *reinterpret_cast<const float4*>(absmax + b);
    acc += (double)v.x;
    acc += (double)v.y;
    acc += (double)v.z;
    acc += (double)v.w;
  }
  for (; b < b1; ++b) acc += (double)absmax[b];
  gsum[g] = acc;
}

// one workgroup: lane c sums chunk c of the group sums, lane 0 the chunks
__global__ __launch_bounds__(kDqcChunks) void dqc_mean_kernel(const double* __restrict__ gsum,
                                                              int64_t groups, int64_t nb,
                                                              float* __restrict__ mean) {
  __shared__ double chunk[kDqcChunks];
  const int c = threadIdx.x;
  const int64_t per = (groups + kDqcChunks - 1) / kDqcChunks;
  const int64_t g0 = c * per, g1 = g0 + per < groups ? g0 + per : groups;
  double acc = 0.0;
  for (int64_t g = g0; g < g1; ++g) acc += gsum[g];
  chunk[c] = acc;
  __syncthreads();
  if (c == 0) {
    double total = 0.0;
    for (int i = 0; i < kDqcChunks; ++i) total += chunk[i];
    *mean = (float)(total / (double)nb);
  }
}

// one wave per group, 4 scales per lane (the layout of double_quant_kernel)
__global__ __launch_bounds__(256) void dqc_code_kernel(const float* __restrict__ absmax,
                                                       int64_t nb,
                                                       const float* __restrict__ mean,
                                                       uint8_t* __restrict__ qscale,
                                                       float* __restrict__ step_out) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t groups = (nb + 255) >> 8;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const float mu = *mean;
  for (int64_t gidx = wave0; gidx < groups; gidx += wstride) {
    const int64_t b0 = (gidx << 8) + 4 * lane;
    float d[4];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[i] = b0 + i < nb ? absmax[b0 + i] - mu : 0.0f;  // blocks past the end count 0
      m = fmaxf(m, fabsf(d[i]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float st = __fdiv_rn(m, 127.0f);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = 0;
      if (st > 0.0f) q = (int)fminf(fmaxf(rintf(__fdiv_rn(d[i], st)), -127.0f), 127.0f);
      packed |= ((uint32_t)q & 0xFFu) << (8 * i);
    }
    if (b0 + 4 <= nb) {
      *reinterpret_cast<uint32_t*>(qscale + b0) = packed;
    } else {
      for (int i = 0; i < 4; ++i)
        if (b0 + i < nb) qscale[b0 + i] = (uint8_t)(packed >> (8 * i));
    }
    if (lane == 0) step_out[gidx] = st;
  }
}

size_t dq_centred_workspace_bytes(int64_t nb) {
  const int64_t groups = (nb + 255) >> 8;
  return (size_t)((groups * 8 + 255) / 256 * 256);
}

hipError_t launch_double_quant_centred(const float* absmax, int64_t nb, uint8_t* qscale,
                                       float* step, float* mean, void* workspace,
                                       hipStream_t s) {
  const int64_t groups = (nb + 255) >> 8;
  double* gsum = static_cast<double*>(workspace);
  hipLaunchKernelGGL(dqc_group_sum_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     s, absmax, nb, gsum);
  hipLaunchKernelGGL(dqc_mean_kernel, dim3(1), dim3(kDqcChunks), 0, s, gsum, groups, nb, mean);
  const int grid = grid_for(groups, 4, 256 * 16);
  hipLaunchKernelGGL(dqc_code_kernel, dim3(grid), dim3(256), 0, s, absmax, nb, mean, qscale,
                     step);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone dequantiser: one lane per 64-weight block (the decode routine
// the GEMMs run on their tiles), 32 code bytes in, 128 bf16 bytes out.
// ---------------------------------------------------------------------------
// DT: the 16-bit output type (Bf16T, or F16T for the fp16 compute type).
template <class DT>
__global__ __launch_bounds__(256) void nf4_dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ qscale,
    const float* __restrict__ step, const float* __restrict__ dq_mean, int64_t nb,
    uint16_t* __restrict__ out, Nf4Levels L) {
  const ScaleFmt fmt = scale_fmt(dq_mean);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
    const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(codes + (b << 5));
    const u32x4_t c0 = cp[0], c1 = cp[1];
    const Nf4Lut lut = nf4_make_lut<DT>(L, nf4_block_scale(qscale[b], step[b >> 8], fmt));
    u32x4_t* op = reinterpret_cast<u32x4_t*>(out + (b << 6));
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = nf4_decode8(lut, c0[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) op[4 + i] = nf4_decode8(lut, c1[i]);
  }
}

hipError_t launch_quantize(const float* w, int64_t n, uint8_t* codes, float* absmax,
                           const Nf4CodeBins& bins, hipStream_t s) {
  const int64_t lanes = (n + 7) >> 3;
  const int grid = grid_for(lanes, 256, 256 * 32);
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3(grid), dim3(256), 0, s, w, n, codes, absmax, bins);
  return hipGetLastError();
}

hipError_t launch_quantize_dq(const float* w, int64_t n, uint8_t* codes, float* absmax,
                              uint8_t* qscale, float* step, const Nf4CodeBins& bins,
                              hipStream_t s) {
  const int64_t groups = (n + 16383) / 16384;
  hipLaunchKernelGGL(nf4_quantize_dq_kernel, dim3((unsigned)groups), dim3(1024), 0, s, w, n, codes,
                     absmax, qscale, step, bins);
  return hipGetLastError();
}

hipError_t launch_double_quant(const float* absmax, int64_t nb, uint8_t* qscale,
                               float* step, hipStream_t s) {
  const int64_t groups = (nb + 255) >> 8;
  const int grid = grid_for(groups, 4, 256 * 16);
  hipLaunchKernelGGL(double_quant_kernel, dim3(grid), dim3(256), 0, s, absmax, nb, qscale, step);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const float* dq_mean, int64_t nb, uint16_t* out, const Nf4Levels& L,
                          hipStream_t s, bool f16) {
  const int grid = grid_for(nb, 256, 256 * 16);
  if (f16)
    hipLaunchKernelGGL(nf4_dequant_kernel<F16T>, dim3(grid), dim3(256), 0, s, codes, qscale, step,
                       dq_mean, nb, out, L);
  else
    hipLaunchKernelGGL(nf4_dequant_kernel<Bf16T>, dim3(grid), dim3(256), 0, s, codes, qscale,
                       step, dq_mean, nb, out, L);
  return hipGetLastError();
}

}  // namespace qlora
