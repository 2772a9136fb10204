// C ABI of the QLoRA linear layer: argument validation, workspace layout and
// kernel dispatch.  Every argument is checked before the first HIP call, so
// invalid calls return a status without touching the GPU.  No C++
// exception crosses the ABI.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <stdexcept>

#include "../../include/qlora.h"
#include "launch.h"
#include "nf4_table.h"

namespace {

using qlora::Nf4Levels;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges; empty ranges never overlap)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

Nf4Levels levels_arg() {
  Nf4Levels L;
  std::memcpy(L.v, qlora::nf4_table().level, sizeof(L.v));
  return L;
}
// The quantiser's bin table (see Nf4CodeBins), built from the thresholds with
// the same fp32 bin function the kernel uses.
qlora::Nf4CodeBins code_bins_arg() {
  const qlora::Nf4Table& t = qlora::nf4_table();
  qlora::Nf4CodeBins B;
  for (int b = 0; b < 64; ++b) {
    B.thr[b] = 2.0f;
    B.base[b] = 0;
  }
  for (int i = 0; i < 15; ++i) {
    const uint32_t b = qlora::nf4_bin(t.threshold[i]);
    if (B.thr[b] != 2.0f) throw std::logic_error("two NF4 thresholds in one bin");
    B.thr[b] = t.threshold[i];
    for (int c = (int)b + 1; c < 64; ++c) B.base[c] += 1;
  }
  return B;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// LoRA dropout drawn in the kernels: the Philox key and stream offset, and
// the threshold t = nearest integer to 65536 p (ties to even; the product
// is exact), so the realised dropout probability is t / 65536.
qlora::PhiloxDrop philox_drop(float p, uint64_t seed, uint64_t offset) {
  qlora::PhiloxDrop d;
  d.k0 = (uint32_t)seed;
  d.k1 = (uint32_t)(seed >> 32);
  d.o0 = (uint32_t)offset;
  d.o1 = (uint32_t)(offset >> 32);
  d.t = (uint32_t)std::nearbyint((double)p * 65536.0);
  return d;
}
float realised_p(const qlora::PhiloxDrop& d) { return (float)((double)d.t / 65536.0); }

int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_EHIP; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t pad32(int64_t M) { return (M + 31) / 32 * 32; }

// Validate the packed-weight descriptor for a GEMM of the given M.
int check_weight(const qlora_nf4_weight* w) {
  if (!w || !w->codes || !w->qscale || !w->dq_step) return QLORA_EINVAL;
  if (w->N <= 0 || w->K <= 0) return QLORA_EINVAL;
  if (w->N % 64 || w->K % 64) return QLORA_ESHAPE;
  if (!aligned16(w->codes) || !aligned16(w->qscale) || !aligned16(w->dq_step)) return QLORA_EALIGN;
  if (w->dq_mean && (reinterpret_cast<uintptr_t>(w->dq_mean) & 3)) return QLORA_EALIGN;
  return QLORA_OK;
}

// Validate a bf16 weight [N, K] of the unquantised layer.
int check_bf16_weight(const uint16_t* W, int64_t N, int64_t K) {
  if (!W) return QLORA_EINVAL;
  if (N <= 0 || K <= 0) return QLORA_EINVAL;
  if (N % 64 || K % 64) return QLORA_ESHAPE;
  if (!aligned16(W)) return QLORA_EALIGN;
  return QLORA_OK;
}

// The kernels address every tensor with 32-bit byte offsets (buffer loads):
// the packed codes and each activation tensor must stay within 2 GiB.
constexpr int64_t kMaxTensorBytes = int64_t{1} << 31;
int check_sizes(int64_t M, int64_t N, int64_t K) {
  if (N / 2 > kMaxTensorBytes / K) return QLORA_ESHAPE;  // codes: N * K / 2 bytes
  if (M > 0 && (N > kMaxTensorBytes / 2 / M || K > kMaxTensorBytes / 2 / M))
    return QLORA_ESHAPE;                                  // x, dy, y, dx: M * (N or K) * 2
  return QLORA_OK;
}

int check_rank(int32_t r) {
  if (r < 0) return QLORA_EINVAL;
  if (r > QLORA_MAX_RANK || r % 8) return QLORA_ESHAPE;
  return QLORA_OK;
}

// The adapter kernels address A [r, K] and B [N, r] (bf16), the hi/lo
// products [M][2r] and their token-contiguous copies [2r][pad32(M)] (bf16)
// with 32-bit buffer offsets as well: each must stay below 2 GiB.
int check_adapter_sizes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (r == 0) return QLORA_OK;
  if (int64_t{2} * r * K >= kMaxTensorBytes || int64_t{2} * r * N >= kMaxTensorBytes ||
      int64_t{4} * r * pad32(M) >= kMaxTensorBytes)
    return QLORA_ESHAPE;
  return QLORA_OK;
}

// ---- workspace layout --------------------------------------------------
struct FwdWs {
  size_t xs_off, xst_off, part_off, ppart_off, total;
  int dsplits;   // k splits of the decode path
  size_t gpart;  // fp32 partials of the fused GEMM's schedule (0: none)
  bool decode;   // few tokens: split-K decode path
};
// decode: the few-token decode path may run (NF4 weight, bf16 compute);
// nf4w: the weight is the NF4 one (the fused GEMM may then take its narrow
// tile, which sizes the partials differently)
FwdWs fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, bool decode = true,
                 bool nf4w = true) {
  FwdWs L{};
  L.decode = decode && M <= qlora::kDecodeMaxM;
  if (M == 0) return L;
  if (L.decode) {
    // with an adapter: the k-split partials of x . A^T, [S][M][r] fp32 (at
    // most 16 x 32 x 256 floats, far inside the 32-bit offsets the kernel
    // uses); without one the decode path needs none
    L.dsplits = qlora::decode_splits(M, N, K, r);
    L.part_off = 0;
    L.total = round_up((size_t)L.dsplits * M * r * sizeof(float), 256);
    return L;
  }
  size_t off = 0;
  if (r > 0) {
    // xs = [hi | lo] of s . x . A^T: [M][2r] bf16, and its token-contiguous copy
    L.xs_off = 0;
    L.xst_off = round_up((size_t)M * 2 * r * sizeof(uint16_t), 256);
    off = round_up(L.xst_off + (size_t)pad32(M) * 2 * r * sizeof(uint16_t), 256);
    // fp32 partials of a split down-projection
    const size_t pp = qlora::lora_proj_partial_bytes(qlora::lora_proj_plan(M, r, K, 0), 0, M, r);
    if (pp > 0) {
      L.ppart_off = off;
      off = round_up(off + pp, 256);
    }
  }
  L.gpart = qlora::gemm_partial_bytes(qlora::gemm_config(M, N, K, nf4w), M, N);
  if (L.gpart > 0) {
    L.part_off = off;
    off = round_up(off + L.gpart, 256);
  }
  L.total = off;
  return L;
}

struct BwdWs {
  size_t xs_off, gs_off, xst_off, gst_off, part_off, mask_off, ppx_off, ppg_off, total;
  size_t gpart;  // fp32 partials of the dX GEMM's schedule (0: none)
};
// nf4w: the weight is the NF4 one (the dX GEMM may then take its narrow
// tile, which sizes the partials differently); mask: room for the keep mask
// [M, K / 8] of a dropout drawn in the kernels
BwdWs bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, bool nf4w = true,
                 bool mask = false) {
  BwdWs L{};
  if (M == 0) return L;
  size_t off = 0;
  if (r > 0) {
    // xs = [hi | lo] of s . x . A^T and gs = [hi | lo] of s . dy . B, [M][2r]
    // bf16 each, and their token-contiguous copies [2r][Mp]
    const size_t pair = (size_t)M * 2 * r * sizeof(uint16_t),
                 pairT = (size_t)pad32(M) * 2 * r * sizeof(uint16_t);
    L.xs_off = 0;
    L.gs_off = round_up(L.xs_off + pair, 256);
    L.xst_off = round_up(L.gs_off + pair, 256);
    L.gst_off = round_up(L.xst_off + pairT, 256);
    off = round_up(L.gst_off + pairT, 256);
    // fp32 partials of the split down-projections (x . A^T, dy . B)
    const qlora::ProjPlan pp = qlora::lora_proj_plan(M, r, K, N);
    const size_t px = qlora::lora_proj_partial_bytes(pp, 0, M, r);
    const size_t pg = qlora::lora_proj_partial_bytes(pp, 1, M, r);
    if (px > 0) {
      L.ppx_off = off;
      off = round_up(off + px, 256);
    }
    if (pg > 0) {
      L.ppg_off = off;
      off = round_up(off + pg, 256);
    }
  }
  L.gpart = qlora::gemm_partial_bytes(qlora::gemm_config(M, K, N, nf4w), M, K);
  if (L.gpart > 0) {
    L.part_off = off;
    off = round_up(off + L.gpart, 256);
  }
  if (mask && r > 0) {
    L.mask_off = off;
    off = round_up(off + (size_t)M * (size_t)(K / 8), 256);
  }
  L.total = off;
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// The base weight of a linear call: the NF4 weight, or a bf16 one (the
// unquantised comparison layer).
struct Wref {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  const uint16_t* wbf;
  int64_t N, K;
  const float* mean = nullptr;  // mean-centred scale format (or null)
  bool nf4() const { return wbf == nullptr; }
  const void* data() const { return nf4() ? static_cast<const void*>(codes) : wbf; }
  size_t bytes() const { return nf4() ? (size_t)N * K / 2 : (size_t)N * K * 2; }
};

// keep (or null) and p: LoRA dropout on the adapter's input
// f16: the fp16 compute type (x, A, B, y in fp16), NF4 weight, no dropout
// src (or null): the workspace comes from src(need) once every argument has
// been validated, instead of from workspace / ws_bytes
// drop (or null): LoRA dropout drawn in the kernels (keep is then null)
int fwd_impl(const Wref* w, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
             int32_t r, float alpha, const uint8_t* keep, float p, uint16_t* y,
             void* workspace, size_t ws_bytes, void* stream, bool f16 = false,
             qlora::WorkspaceSource src = nullptr, const qlora::PhiloxDrop* drop = nullptr) {
  try {
    int st = QLORA_OK;
    if ((st = check_rank(r)) != QLORA_OK) return st;
    if ((keep || drop) && !(p >= 0.0f && p < 1.0f)) return QLORA_EINVAL;
    if (r == 0) {
      keep = nullptr;
      drop = nullptr;
    }
    if (M < 0) return QLORA_EINVAL;
    const int64_t N = w->N, K = w->K;
    if ((st = check_sizes(M, N, K)) != QLORA_OK) return st;
    if ((st = check_adapter_sizes(M, N, K, r)) != QLORA_OK) return st;
    if (M == 0) return QLORA_OK;
    if (!x || !y) return QLORA_EINVAL;
    if (r > 0 && (!A || !B)) return QLORA_EINVAL;
    if (!aligned16(x) || !aligned16(y) || (r > 0 && (!aligned16(A) || !aligned16(B))) ||
        (keep && !aligned16(keep)))
      return QLORA_EALIGN;
    // the few-token decode kernel computes in bf16 only: with fp16 the
    // tiled path runs
    const FwdWs ws = fwd_layout(M, N, K, r, w->nf4() && !f16, w->nf4());
    const size_t ny = (size_t)M * N * 2;
    if (overlap(y, ny, x, (size_t)M * K * 2) || overlap(y, ny, w->data(), w->bytes()) ||
        (r > 0 && (overlap(y, ny, A, (size_t)r * K * 2) || overlap(y, ny, B, (size_t)N * r * 2))) ||
        (keep && overlap(y, ny, keep, (size_t)M * K / 8)))
      return QLORA_EINVAL;
    if (src && ws.total > 0) {
      workspace = src(ws.total, &st);
      if (!workspace) return st;
      ws_bytes = ws.total;
    }
    if (ws.total > 0) {
      if (!workspace || ws_bytes < ws.total) return QLORA_EWORKSPACE;
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QLORA_EALIGN;
      if (overlap(y, ny, workspace, ws.total)) return QLORA_EINVAL;
    }

    hipStream_t s = as_stream(stream);
    const Nf4Levels L = levels_arg();
    // inverted dropout: the kept values are scaled by 1 / (1 - p), folded
    // into s (a drawn dropout realises p as t / 65536)
    const float pd = drop ? realised_p(*drop) : p;
    const float scale =
        r > 0 ? alpha / static_cast<float>(r) / (keep || drop ? 1.0f - pd : 1.0f) : 0.0f;
    if (ws.decode) {
      return hip_status(qlora::launch_decode_fwd(
          w->codes, w->qscale, w->step, w->mean, x, A, B, r, scale,
          ws.total > 0 ? at<float>(workspace, ws.part_off) : nullptr, ws.dsplits, y, M, N, K, L,
          s, keep, drop));
    }
    uint16_t* xs = nullptr;
    if (r > 0) {
      xs = at<uint16_t>(workspace, ws.xs_off);
      qlora::LoraProjJob jx{x, A, xs, at<uint16_t>(workspace, ws.xst_off), K, 0, keep};
      if (drop) {
        jx.rng = 1;
        jx.drop = *drop;
      }
      if (ws.ppart_off) jx.part = at<float>(workspace, ws.ppart_off);
      if ((st = hip_status(qlora::launch_lora_proj(jx, nullptr, M, r, scale, s, f16))) !=
          QLORA_OK)
        return st;
    }
    float* part = ws.gpart > 0 ? at<float>(workspace, ws.part_off) : nullptr;
    return hip_status(qlora::launch_fwd_gemm(w->codes, w->qscale, w->step, w->mean, w->wbf, x, xs, B, y,
                                             part, M, N, K, r, L, s, f16));
  } catch (...) {
    return QLORA_EHIP;
  }
}

// drop (or null): LoRA dropout drawn in the kernels (keep is then null): the
// down-projection draws the keep bits and stores them in the workspace, where
// the gradient and dX kernels read them as a passed-in mask
int bwd_impl(const Wref* w, const uint16_t* x, const uint16_t* dy, int64_t M, const uint16_t* A,
             const uint16_t* B, int32_t r, float alpha, const uint8_t* keep, float p,
             uint16_t* dx, float* dA, float* dB, int32_t accumulate, void* workspace,
             size_t ws_bytes, void* stream, bool f16 = false,
             const qlora::PhiloxDrop* drop = nullptr) {
  try {
    int st = QLORA_OK;
    if ((st = check_rank(r)) != QLORA_OK) return st;
    if ((keep || drop) && !(p >= 0.0f && p < 1.0f)) return QLORA_EINVAL;
    if (r == 0) {
      keep = nullptr;
      drop = nullptr;
    }
    if (M < 0) return QLORA_EINVAL;
    const int64_t N = w->N, K = w->K;
    if ((st = check_sizes(M, N, K)) != QLORA_OK) return st;
    if ((st = check_adapter_sizes(M, N, K, r)) != QLORA_OK) return st;
    if (M == 0) {
      // a sum over no tokens: dA = dB = 0 (or unchanged when accumulating)
      if (r == 0) return QLORA_OK;
      if (!dA || !dB) return QLORA_EINVAL;
      if (!aligned16(dA) || !aligned16(dB)) return QLORA_EALIGN;
      if (overlap(dA, (size_t)r * K * 4, dB, (size_t)N * r * 4)) return QLORA_EINVAL;
      // the gradient kernel with no tokens writes zeros (or adds nothing)
      const qlora::LoraGradJob jb{nullptr, nullptr, dB, N, 0}, ja{nullptr, nullptr, dA, K, 1};
      return hip_status(
          qlora::launch_lora_grad(jb, ja, 0, r, accumulate, as_stream(stream), f16));
    }
    if (!dy) return QLORA_EINVAL;
    if (r > 0 && (!A || !B || !x || !dA || !dB)) return QLORA_EINVAL;
    if (!aligned16(dy) || (dx && !aligned16(dx)) ||
        (r > 0 && (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(dA) ||
                   !aligned16(dB))) ||
        (keep && !aligned16(keep)))
      return QLORA_EALIGN;
    const BwdWs ws = bwd_layout(M, N, K, r, w->nf4(), drop != nullptr);
    if (ws.total > 0) {
      if (!workspace || ws_bytes < ws.total) return QLORA_EWORKSPACE;
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return QLORA_EALIGN;
    }
    // outputs must not overlap inputs, the workspace or each other
    const size_t nxb = (size_t)M * K * 2, nyb = (size_t)M * N * 2, nab = (size_t)r * K * 4,
                 nbb = (size_t)N * r * 4;
    const void* ins[] = {x, dy, A, B, w->data(), workspace, keep};
    const size_t in_sz[] = {nxb, nyb, (size_t)r * K * 2, (size_t)N * r * 2, w->bytes(),
                            ws.total, keep ? (size_t)M * K / 8 : 0};
    void* outs[] = {dx, r > 0 ? dA : nullptr, r > 0 ? dB : nullptr};
    const size_t out_sz[] = {nxb, nab, nbb};
    for (int o = 0; o < 3; ++o) {
      for (int i = 0; i < 7; ++i)
        if (overlap(outs[o], out_sz[o], ins[i], in_sz[i])) return QLORA_EINVAL;
      for (int o2 = o + 1; o2 < 3; ++o2)
        if (overlap(outs[o], out_sz[o], outs[o2], out_sz[o2])) return QLORA_EINVAL;
    }
    hipStream_t s = as_stream(stream);

    const Nf4Levels L = levels_arg();
    uint16_t* gs = nullptr;
    if (r > 0) {
      uint16_t* xs = at<uint16_t>(workspace, ws.xs_off);
      gs = at<uint16_t>(workspace, ws.gs_off);
      // with dropout, s / (1 - p): dB, dA and dX's adapter term all carry it
      // (a drawn dropout realises p as t / 65536)
      const float pd = drop ? realised_p(*drop) : p;
      const float scale =
          alpha / static_cast<float>(r) / (keep || drop ? 1.0f - pd : 1.0f);
      // xs = split(s . x~ . A^T), gs = split(s . dy . B) in one launch (x~:
      // x with the dropped values zeroed)
      uint16_t* xsT = at<uint16_t>(workspace, ws.xst_off);
      uint16_t* gsT = at<uint16_t>(workspace, ws.gst_off);
      qlora::LoraProjJob jx{x, A, xs, xsT, K, 0, keep}, jg{dy, B, gs, gsT, N, 1, nullptr};
      if (ws.ppx_off) jx.part = at<float>(workspace, ws.ppx_off);
      if (ws.ppg_off) jg.part = at<float>(workspace, ws.ppg_off);
      if (drop) {
        // drawn here once; dA and dX read the stored bytes
        jx.rng = 1;
        jx.drop = *drop;
        jx.keep_out = at<uint8_t>(workspace, ws.mask_off);
        keep = jx.keep_out;
      }
      if ((st = hip_status(qlora::launch_lora_proj(jx, &jg, M, r, scale, s, f16))) != QLORA_OK)
        return st;
      // dB [N, r] = dy^T . (xs_hi + xs_lo);  dA [r, K] = (gs_hi + gs_lo)^T . x~
      const qlora::LoraGradJob jb{dy, xsT, dB, N, 0, nullptr}, ja{x, gsT, dA, K, 1, keep};
      if ((st = hip_status(qlora::launch_lora_grad(jb, ja, M, r, accumulate, s, f16))) !=
          QLORA_OK)
        return st;
    }
    if (dx) {
      float* part = ws.gpart > 0 ? at<float>(workspace, ws.part_off) : nullptr;
      if ((st = hip_status(qlora::launch_dx_gemm(w->codes, w->qscale, w->step, w->mean, w->wbf, keep, dy, gs,
                                                 A, dx, part, M, N, K, r, L, s, f16))) != QLORA_OK)
        return st;
    }
    return QLORA_OK;
  } catch (...) {
    return QLORA_EHIP;
  }
}

}  // namespace

namespace qlora {

int linear_fwd_sourced(const qlora_nf4_weight* w, const uint16_t* x, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float alpha, uint16_t* y,
                       WorkspaceSource src, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return fwd_impl(&wr, x, M, A, B, r, alpha, nullptr, 0.0f, y, nullptr, 0, stream, false, src);
}

}  // namespace qlora

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument (null pointer, negative size or aliasing)";
    case QLORA_ESHAPE:
      return "unsupported shape (N, K must be multiples of 64; r a multiple of 8 <= 256; "
             "codes, each activation tensor, A, B and the adapter products below 2 GiB)";
    case QLORA_EALIGN: return "device pointer not 16-byte aligned";
    case QLORA_ENOTSUP: return "unsupported block size (64 / 256 only)";
    case QLORA_EWORKSPACE: return "workspace missing or too small";
    case QLORA_EHIP: return "HIP launch or runtime error";
    case QLORA_ESCRATCH:
      return "the call needs more scratch than the library's static buffer holds "
             "(QLORA_NOALLOC_SCRATCH_BYTES); use the call with a caller workspace";
    default: return "unknown status";
  }
}

int qlora_nf4_levels(float out[16]) {
  if (!out) return QLORA_EINVAL;
  try {
    const qlora::Nf4Table& t = qlora::nf4_table();
    std::memcpy(out, t.level, sizeof(t.level));
    return QLORA_OK;
  } catch (...) {
    return QLORA_EINVAL;
  }
}

int qlora_nf4_thresholds(float out[15]) {
  if (!out) return QLORA_EINVAL;
  try {
    const qlora::Nf4Table& t = qlora::nf4_table();
    std::memcpy(out, t.threshold, sizeof(t.threshold));
    return QLORA_OK;
  } catch (...) {
    return QLORA_EINVAL;
  }
}

size_t qlora_linear_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64 || check_rank(r) != QLORA_OK ||
      check_sizes(M, N, K) != QLORA_OK || check_adapter_sizes(M, N, K, r) != QLORA_OK)
    return 0;
  if (op == 0) return fwd_layout(M, N, K, r).total;
  if (op == 1) return bwd_layout(M, N, K, r).total;
  if (op == 3) return bwd_layout(M, N, K, r, false).total;
  if (op == 2) return fwd_layout(M, N, K, r, false, false).total;
  if (op == 4) return fwd_layout(M, N, K, r, true, true).total;
  if (op == 6) return fwd_layout(M, N, K, r, false, true).total;
  if (op == 5 || op == 7) return bwd_layout(M, N, K, r).total;
  if (op == 8) return fwd_layout(M, N, K, r, true, true).total;
  if (op == 9) return bwd_layout(M, N, K, r, true, true).total;
  return 0;
}

int qlora_dropout_keep_mask(int64_t M, int64_t K, float p, uint64_t seed, uint64_t offset,
                            uint8_t* keep, void* stream) {
  try {
    if (M < 0 || K <= 0) return QLORA_EINVAL;
    if (!(p >= 0.0f && p < 1.0f)) return QLORA_EINVAL;
    if (K % 8) return QLORA_ESHAPE;
    // the activation the mask belongs to is at most 2 GiB of bf16
    if (M > 0 && K > kMaxTensorBytes / 2 / M) return QLORA_ESHAPE;
    if (M == 0) return QLORA_OK;
    if (!keep) return QLORA_EINVAL;
    if (!aligned16(keep)) return QLORA_EALIGN;
    return hip_status(
        qlora::launch_dropout_mask(philox_drop(p, seed, offset), M, K, keep, as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

int qlora_linear_fwd_dropout_rng(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                                 const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                                 float p, uint64_t seed, uint64_t offset, uint16_t* y,
                                 void* workspace, size_t ws_bytes, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  const qlora::PhiloxDrop d = philox_drop(p, seed, offset);
  return fwd_impl(&wr, x, M, A, B, r, alpha, nullptr, p, y, workspace, ws_bytes, stream, false,
                  nullptr, &d);
}

int qlora_linear_bwd_dropout_rng(const qlora_nf4_weight* w, const uint16_t* x,
                                 const uint16_t* dy, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float alpha, float p,
                                 uint64_t seed, uint64_t offset, uint16_t* dx, float* dA,
                                 float* dB, int32_t accumulate, void* workspace, size_t ws_bytes,
                                 void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  const qlora::PhiloxDrop d = philox_drop(p, seed, offset);
  return bwd_impl(&wr, x, dy, M, A, B, r, alpha, nullptr, p, dx, dA, dB, accumulate, workspace,
                  ws_bytes, stream, false, &d);
}

int qlora_quantize_nf4(const float* w, int64_t n_elems, int32_t blocksize, uint8_t* codes,
                       float* absmax, void* stream) {
  try {
    if (n_elems < 0) return QLORA_EINVAL;
    if (blocksize != QLORA_BLOCK) return QLORA_ENOTSUP;
    if (n_elems == 0) return QLORA_OK;
    if (!w || !codes || !absmax) return QLORA_EINVAL;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax)) return QLORA_EALIGN;
    const size_t nw = (size_t)n_elems * 4, nc = (size_t)(n_elems + 1) / 2,
                 na = (size_t)((n_elems + 63) / 64) * 4;
    if (overlap(w, nw, codes, nc) || overlap(w, nw, absmax, na) || overlap(codes, nc, absmax, na))
      return QLORA_EINVAL;
    return hip_status(qlora::launch_quantize(w, n_elems, codes, absmax, code_bins_arg(),
                                             as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

int qlora_double_quant(const float* absmax, int64_t n_blocks, int32_t blocksize2,
                       uint8_t* qscale, float* dq_step, void* stream) {
  try {
    if (n_blocks < 0) return QLORA_EINVAL;
    if (blocksize2 != QLORA_GROUP) return QLORA_ENOTSUP;
    if (n_blocks == 0) return QLORA_OK;
    if (!absmax || !qscale || !dq_step) return QLORA_EINVAL;
    if (!aligned16(absmax) || !aligned16(qscale) || !aligned16(dq_step)) return QLORA_EALIGN;
    const size_t na = (size_t)n_blocks * 4, nq = (size_t)n_blocks,
                 ns = (size_t)((n_blocks + 255) / 256) * 4;
    if (overlap(absmax, na, qscale, nq) || overlap(absmax, na, dq_step, ns) ||
        overlap(qscale, nq, dq_step, ns))
      return QLORA_EINVAL;
    return hip_status(qlora::launch_double_quant(absmax, n_blocks, qscale, dq_step,
                                                 as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

int qlora_quantize_nf4_dq(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                          uint8_t* qscale, float* dq_step, void* stream) {
  try {
    if (n_elems < 0) return QLORA_EINVAL;
    if (n_elems == 0) return QLORA_OK;
    if (!w || !codes || !absmax || !qscale || !dq_step) return QLORA_EINVAL;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax) || !aligned16(qscale) ||
        !aligned16(dq_step))
      return QLORA_EALIGN;
    const int64_t nb = (n_elems + 63) / 64;
    const size_t nw = (size_t)n_elems * 4, nc = (size_t)(n_elems + 1) / 2, na = (size_t)nb * 4,
                 nq = (size_t)nb, ns = (size_t)((nb + 255) / 256) * 4;
    const void* p[5] = {w, codes, absmax, qscale, dq_step};
    const size_t sz[5] = {nw, nc, na, nq, ns};
    for (int i = 0; i < 5; ++i)
      for (int j = i + 1; j < 5; ++j)
        if (overlap(p[i], sz[i], p[j], sz[j])) return QLORA_EINVAL;
    return hip_status(qlora::launch_quantize_dq(w, n_elems, codes, absmax, qscale, dq_step,
                                                code_bins_arg(), as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

size_t qlora_dq_centred_workspace_bytes(int64_t n_blocks) {
  return n_blocks > 0 ? qlora::dq_centred_workspace_bytes(n_blocks) : 0;
}

// the checks shared by the two mean-centred entry points (absmax and the
// outputs of the scale encoding)
static int check_dq_centred(const float* absmax, int64_t nb, const uint8_t* qscale,
                            const float* dq_step, const float* dq_mean, void* workspace,
                            size_t ws_bytes) {
  if (!absmax || !qscale || !dq_step || !dq_mean || !workspace) return QLORA_EINVAL;
  if (!aligned16(absmax) || !aligned16(qscale) || !aligned16(dq_step) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(dq_mean) & 3))
    return QLORA_EALIGN;
  if (ws_bytes < qlora::dq_centred_workspace_bytes(nb)) return QLORA_EWORKSPACE;
  const size_t ns = (size_t)((nb + 255) / 256) * 4, nw = qlora::dq_centred_workspace_bytes(nb);
  const void* p[5] = {absmax, qscale, dq_step, dq_mean, workspace};
  const size_t sz[5] = {(size_t)nb * 4, (size_t)nb, ns, 4, nw};
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(p[i], sz[i], p[j], sz[j])) return QLORA_EINVAL;
  return QLORA_OK;
}

int qlora_double_quant_centred(const float* absmax, int64_t n_blocks, uint8_t* qscale,
                               float* dq_step, float* dq_mean, void* workspace, size_t ws_bytes,
                               void* stream) {
  try {
    if (n_blocks < 0) return QLORA_EINVAL;
    if (n_blocks == 0) return QLORA_OK;
    const int st = check_dq_centred(absmax, n_blocks, qscale, dq_step, dq_mean, workspace,
                                    ws_bytes);
    if (st != QLORA_OK) return st;
    return hip_status(qlora::launch_double_quant_centred(absmax, n_blocks, qscale, dq_step,
                                                         dq_mean, workspace, as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

int qlora_quantize_nf4_dq_centred(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                                  uint8_t* qscale, float* dq_step, float* dq_mean,
                                  void* workspace, size_t ws_bytes, void* stream) {
  try {
    if (n_elems < 0) return QLORA_EINVAL;
    if (n_elems == 0) return QLORA_OK;
    if (!w || !codes) return QLORA_EINVAL;
    if (!aligned16(w) || !aligned16(codes)) return QLORA_EALIGN;
    const int64_t nb = (n_elems + 63) / 64;
    int st = check_dq_centred(absmax, nb, qscale, dq_step, dq_mean, workspace, ws_bytes);
    if (st != QLORA_OK) return st;
    const size_t nw = (size_t)n_elems * 4, nc = (size_t)(n_elems + 1) / 2;
    const void* outs[6] = {codes, absmax, qscale, dq_step, dq_mean, workspace};
    const size_t osz[6] = {nc, (size_t)nb * 4, (size_t)nb, (size_t)((nb + 255) / 256) * 4, 4,
                           qlora::dq_centred_workspace_bytes(nb)};
    for (int i = 0; i < 6; ++i) {
      if (overlap(w, nw, outs[i], osz[i])) return QLORA_EINVAL;
      if (i > 0 && overlap(codes, nc, outs[i], osz[i])) return QLORA_EINVAL;
    }
    hipStream_t s = as_stream(stream);
    if ((st = hip_status(qlora::launch_quantize(w, n_elems, codes, absmax, code_bins_arg(), s))) !=
        QLORA_OK)
      return st;
    return hip_status(
        qlora::launch_double_quant_centred(absmax, nb, qscale, dq_step, dq_mean, workspace, s));
  } catch (...) {
    return QLORA_EHIP;
  }
}

static int dequantize_impl(const qlora_nf4_weight* w, uint16_t* out, void* stream, bool f16) {
  try {
    if (!w || !w->codes || !w->qscale || !w->dq_step || !out) return QLORA_EINVAL;
    if (w->N <= 0 || w->K <= 0) return QLORA_EINVAL;
    const int64_t n = w->N * w->K;
    if (n % 64) return QLORA_ESHAPE;
    if (!aligned16(w->codes) || !aligned16(w->qscale) || !aligned16(w->dq_step) ||
        !aligned16(out))
      return QLORA_EALIGN;
    const size_t no = (size_t)n * 2;
    if (overlap(out, no, w->codes, (size_t)n / 2) || overlap(out, no, w->qscale, (size_t)n / 64))
      return QLORA_EINVAL;
    if (w->dq_mean && (reinterpret_cast<uintptr_t>(w->dq_mean) & 3)) return QLORA_EALIGN;
    return hip_status(qlora::launch_dequant(w->codes, w->qscale, w->dq_step, w->dq_mean, n / 64,
                                            out, levels_arg(), as_stream(stream), f16));
  } catch (...) {
    return QLORA_EHIP;
  }
}

int qlora_dequantize_nf4(const qlora_nf4_weight* w, uint16_t* out, void* stream) {
  return dequantize_impl(w, out, stream, false);
}

int qlora_dequantize_nf4_f16(const qlora_nf4_weight* w, uint16_t* out, void* stream) {
  return dequantize_impl(w, out, stream, true);
}

int qlora_linear_fwd_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                         const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                         uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return fwd_impl(&wr, x, M, A, B, r, alpha, nullptr, 0.0f, y, workspace, ws_bytes, stream,
                  true);
}

int qlora_linear_bwd_f16(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                         int64_t M, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                         uint16_t* dx, float* dA, float* dB, int32_t accumulate, void* workspace,
                         size_t ws_bytes, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return bwd_impl(&wr, x, dy, M, A, B, r, alpha, nullptr, 0.0f, dx, dA, dB, accumulate,
                  workspace, ws_bytes, stream, true);
}

int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* x, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, uint16_t* y, void* workspace,
                     size_t ws_bytes, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return fwd_impl(&wr, x, M, A, B, r, alpha, nullptr, 0.0f, y, workspace, ws_bytes, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha, uint16_t* dx,
                     float* dA, float* dB, int32_t accumulate, void* workspace, size_t ws_bytes,
                     void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return bwd_impl(&wr, x, dy, M, A, B, r, alpha, nullptr, 0.0f, dx, dA, dB, accumulate,
                  workspace, ws_bytes, stream);
}

int qlora_linear_bf16_fwd(const uint16_t* W, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                          const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                          uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  const int st = check_bf16_weight(W, N, K);
  if (st != QLORA_OK) return st;
  const Wref wr{nullptr, nullptr, nullptr, W, N, K};
  return fwd_impl(&wr, x, M, A, B, r, alpha, nullptr, 0.0f, y, workspace, ws_bytes, stream);
}

int qlora_linear_bf16_bwd(const uint16_t* W, int64_t N, int64_t K, const uint16_t* x,
                          const uint16_t* dy, int64_t M, const uint16_t* A, const uint16_t* B,
                          int32_t r, float alpha, uint16_t* dx, float* dA, float* dB,
                          int32_t accumulate, void* workspace, size_t ws_bytes, void* stream) {
  const int st = check_bf16_weight(W, N, K);
  if (st != QLORA_OK) return st;
  const Wref wr{nullptr, nullptr, nullptr, W, N, K};
  return bwd_impl(&wr, x, dy, M, A, B, r, alpha, nullptr, 0.0f, dx, dA, dB, accumulate,
                  workspace, ws_bytes, stream);
}

int qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                             const uint8_t* keep, float p, uint16_t* y, void* workspace,
                             size_t ws_bytes, void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  if (!keep) return QLORA_EINVAL;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return fwd_impl(&wr, x, M, A, B, r, alpha, keep, p, y, workspace, ws_bytes, stream);
}

int qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                             int64_t M, const uint16_t* A, const uint16_t* B, int32_t r,
                             float alpha, const uint8_t* keep, float p, uint16_t* dx, float* dA,
                             float* dB, int32_t accumulate, void* workspace, size_t ws_bytes,
                             void* stream) {
  const int st = check_weight(w);
  if (st != QLORA_OK) return st;
  if (!keep) return QLORA_EINVAL;
  const Wref wr{w->codes, w->qscale, w->dq_step, nullptr, w->N, w->K, w->dq_mean};
  return bwd_impl(&wr, x, dy, M, A, B, r, alpha, keep, p, dx, dA, dB, accumulate, workspace,
                  ws_bytes, stream);
}

int qlora_merge_adapter(const qlora_nf4_weight* w, const float* w0, int64_t N, int64_t K,
                        const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                        float* out_f32, uint16_t* out_bf16, void* stream) {
  try {
    if ((w == nullptr) == (w0 == nullptr)) return QLORA_EINVAL;
    if (!out_f32 && !out_bf16) return QLORA_EINVAL;
    int st = check_rank(r);
    if (st != QLORA_OK) return st;
    if (N <= 0 || K <= 0) return QLORA_EINVAL;
    if (w) {
      if ((st = check_weight(w)) != QLORA_OK) return st;
      if (w->N != N || w->K != K) return QLORA_ESHAPE;
    }
    if (N % 64 || K % 64) return QLORA_ESHAPE;
    // B is read through 32-bit buffer offsets; everything else is addressed
    // with 64-bit pointers (N * K bounded only to keep the sizes below exact)
    if (N * r * 2 >= kMaxTensorBytes || N > (int64_t{1} << 40) / K) return QLORA_ESHAPE;
    if (r > 0 && (!A || !B)) return QLORA_EINVAL;
    if ((w0 && !aligned16(w0)) || (out_f32 && !aligned16(out_f32)) ||
        (out_bf16 && !aligned16(out_bf16)) || (r > 0 && (!aligned16(A) || !aligned16(B))))
      return QLORA_EALIGN;
    const size_t n = (size_t)N * (size_t)K;
    const size_t nf = out_f32 ? n * 4 : 0, nb = out_bf16 ? n * 2 : 0;
    const size_t na = r > 0 ? (size_t)r * K * 2 : 0, nB = r > 0 ? (size_t)N * r * 2 : 0;
    const void* ins[5] = {w0, A, B, w ? w->codes : nullptr, w ? w->qscale : nullptr};
    const size_t in_bytes[5] = {w0 ? n * 4 : 0, na, nB, w ? n / 2 : 0, w ? n / 64 : 0};
    for (int i = 0; i < 5; ++i)
      if (overlap(out_f32, nf, ins[i], in_bytes[i]) || overlap(out_bf16, nb, ins[i], in_bytes[i]))
        return QLORA_EINVAL;
    if (w && (overlap(out_f32, nf, w->dq_step, (n / 64 + 255) / 256 * 4) ||
              overlap(out_bf16, nb, w->dq_step, (n / 64 + 255) / 256 * 4)))
      return QLORA_EINVAL;
    if (overlap(out_f32, nf, out_bf16, nb)) return QLORA_EINVAL;
    const float scale = r > 0 ? alpha / (float)r : 0.0f;
    return hip_status(qlora::launch_merge(w ? w->codes : nullptr, w ? w->qscale : nullptr,
                                          w ? w->dq_step : nullptr,
                                          w ? w->dq_mean : nullptr, w0, A, B, r, scale,
                                          out_f32, out_bf16, N, K, levels_arg(),
                                          as_stream(stream)));
  } catch (...) {
    return QLORA_EHIP;
  }
}

}  // extern "C"
