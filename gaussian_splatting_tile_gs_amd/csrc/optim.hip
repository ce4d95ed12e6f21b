// Optimizer step: Adam on the raw (unconstrained) parameters, the step that follows the backward
// in the fitting loop of "Gaussian splatting in PyTorch" (section 7, torch.optim.Adam, with the
// per-parameter learning rates it lists for 3DGS training), plus the splat-size penalty of "The
// backward pass I deleted" (the distillation loss's extra term; its form, not given there, is
// lambda * mean over Gaussians of sum_j exp(l_j), so dL/dl_j gains lambda exp(l_j) / n).
//
// Adam (Kingma and Ba 2015, in torch.optim.Adam's order): m <- b1 m + (1 - b1) g,
// v <- b2 v + (1 - b2) g^2, p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps).
// Elementwise and HBM-bound: 16 B read and 12 B written per parameter. One launch covers the
// five parameter groups (blockIdx.y), each a contiguous array, so every wave reads and writes
// consecutive addresses of one group, four values per lane (float4) where the group's arrays
// allow it. The moments of each group start on a 64-float boundary so that they always do.
#include "gs_internal.h"

#include <cmath>

namespace gs {
namespace {

constexpr int kAdamThreads = 256;
constexpr int kAdamBlocks = 2048;  // per group; a grid-stride loop covers the rest
constexpr int kAdamGroups = 5;
constexpr uint64_t kAdamStateAlign = 64;  // floats: every group's moments start 256-byte aligned

struct AdamSeg {
  float* p;
  const float* g;
  float* m;
  float* v;
  uint32_t count;
  uint32_t period;  // SH: 3K values per Gaussian, the first 3 of which are band 0; else 0
  uint32_t vec;     // count % 4 == 0 and all four arrays 16-byte aligned: float4 path
  float lr;         // the group's learning rate (SH: band 0)
  float lr_alt;     // SH: bands >= 1
  float penalty;    // log-scales: lambda / n of the size penalty; else 0
};

struct AdamArgs {
  AdamSeg seg[kAdamGroups];
  float b1, b2, eps, step_scale, inv_sqrt_bc2;  // step_scale = 1 / (1 - b1^t)
};

__device__ __forceinline__ void adam_value(float& p, float g, float& m, float& v, float lr, float penalty,
                                           const AdamArgs& a) {
  if (penalty != 0.0f) g = fmaf(penalty, expf(p), g);
  m = fmaf(a.b1, m, (1.0f - a.b1) * g);
  v = fmaf(a.b2, v, (1.0f - a.b2) * (g * g));
  const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
  p = p - (lr * a.step_scale) * m / denom;
}

__global__ __launch_bounds__(kAdamThreads) void k_adam(AdamArgs a) {
  const AdamSeg& sg = a.seg[blockIdx.y];
  const uint32_t stride = gridDim.x * kAdamThreads;
  const uint32_t first = blockIdx.x * kAdamThreads + threadIdx.x;
  if (sg.vec) {
    float4* p4 = reinterpret_cast<float4*>(sg.p);
    const float4* g4 = reinterpret_cast<const float4*>(sg.g);
    float4* m4 = reinterpret_cast<float4*>(sg.m);
    float4* v4 = reinterpret_cast<float4*>(sg.v);
    for (uint32_t q = first; q < sg.count / 4; q += stride) {
      float4 p = p4[q], m = m4[q], v = v4[q];
      const float4 g = g4[q];
      // position inside the Gaussian's SH block of the first of the four values
      uint32_t r = sg.period ? (4 * q) % sg.period : 0;
      float* pp = &p.x;
      float* mm = &m.x;
      float* vv = &v.x;
      const float* gg = &g.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lr = (sg.period != 0 && r >= 3u) ? sg.lr_alt : sg.lr;
        adam_value(pp[j], gg[j], mm[j], vv[j], lr, sg.penalty, a);
        r = (r + 1 == sg.period) ? 0 : r + 1;
      }
      p4[q] = p;
      m4[q] = m;
      v4[q] = v;
    }
  } else {
    for (uint32_t i = first; i < sg.count; i += stride) {
      float p = sg.p[i], m = sg.m[i], v = sg.v[i];
      const float lr = (sg.period != 0 && i % sg.period >= 3u) ? sg.lr_alt : sg.lr;
      adam_value(p, sg.g[i], m, v, lr, sg.penalty, a);
      sg.p[i] = p;
      sg.m[i] = m;
      sg.v[i] = v;
    }
  }
}

uint64_t group_counts(uint64_t n, int sh_degree, uint64_t cnt[kAdamGroups]) {
  const uint64_t K3 = 3ull * (uint64_t)((sh_degree + 1) * (sh_degree + 1));
  cnt[0] = 3 * n;
  cnt[1] = 3 * n;
  cnt[2] = 4 * n;
  cnt[3] = n;
  cnt[4] = K3 * n;
  return K3;
}

uint64_t padded(uint64_t c) { return (c + kAdamStateAlign - 1) / kAdamStateAlign * kAdamStateAlign; }

bool finite_pos(float x) { return std::isfinite(x) && x >= 0.0f; }

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_adam_state_floats(int32_t n, int32_t sh_degree) {
  if (n <= 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return 0;
  uint64_t cnt[kAdamGroups];
  group_counts((uint64_t)n, sh_degree, cnt);
  uint64_t total = 0;
  for (int k = 0; k < kAdamGroups; ++k) total += padded(cnt[k]);
  return (size_t)total;
}

extern "C" gs_status gs_adam_step(int32_t n, int32_t sh_degree, int32_t step, const gs_adam_config* cfg,
                                  float* d_means, float* d_log_scales, float* d_quats, float* d_opacity_logits,
                                  float* d_sh, const float* d_grad_means, const float* d_grad_log_scales,
                                  const float* d_grad_quats, const float* d_grad_opacity_logits,
                                  const float* d_grad_sh, float* d_m, float* d_v, void* stream) {
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, "gs_adam_step: n < 0");
  if (sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE)
    return set_error(GS_ERR_INVALID_ARG, "gs_adam_step: sh_degree not in 0..3");
  if (step < 1) return set_error(GS_ERR_INVALID_ARG, "gs_adam_step: step < 1");
  if (!cfg) return set_error(GS_ERR_INVALID_ARG, "gs_adam_step: NULL config");
  if (!finite_pos(cfg->lr_means) || !finite_pos(cfg->lr_log_scales) || !finite_pos(cfg->lr_quats) ||
      !finite_pos(cfg->lr_opacity) || !finite_pos(cfg->lr_sh_dc) || !finite_pos(cfg->lr_sh_rest) ||
      !finite_pos(cfg->size_penalty) || !(cfg->beta1 >= 0.0f && cfg->beta1 < 1.0f) ||
      !(cfg->beta2 >= 0.0f && cfg->beta2 < 1.0f) || !(std::isfinite(cfg->eps) && cfg->eps > 0.0f))
    return set_error(GS_ERR_INVALID_ARG,
                     "gs_adam_step: learning rates and penalty must be finite and >= 0, betas in [0, 1), eps > 0");
  if (n == 0) return GS_OK;
  if (!d_means || !d_log_scales || !d_quats || !d_opacity_logits || !d_sh || !d_grad_means || !d_grad_log_scales ||
      !d_grad_quats || !d_grad_opacity_logits || !d_grad_sh || !d_m || !d_v)
    return set_error(GS_ERR_INVALID_ARG, "gs_adam_step: NULL pointer with n > 0");
  uint64_t cnt[kAdamGroups];
  const uint64_t K3 = group_counts((uint64_t)n, sh_degree, cnt);
  // 32-bit indices: a grid-stride step past 2^31 values still fits
  if (cnt[4] >= (1ull << 31)) return set_error(GS_ERR_LIMIT, "gs_adam_step: 3 K n >= 2^31 SH values");
  AdamArgs a{};
  float* P[kAdamGroups] = {d_means, d_log_scales, d_quats, d_opacity_logits, d_sh};
  const float* G[kAdamGroups] = {d_grad_means, d_grad_log_scales, d_grad_quats, d_grad_opacity_logits, d_grad_sh};
  const float lr[kAdamGroups] = {cfg->lr_means, cfg->lr_log_scales, cfg->lr_quats, cfg->lr_opacity, cfg->lr_sh_dc};
  uint64_t off = 0, most = 0;
  for (int k = 0; k < kAdamGroups; ++k) {
    AdamSeg& sg = a.seg[k];
    sg = AdamSeg{P[k], G[k], d_m + off, d_v + off, (uint32_t)cnt[k], 0u, 0u, lr[k], lr[k], 0.0f};
    const uintptr_t al = reinterpret_cast<uintptr_t>(sg.p) | reinterpret_cast<uintptr_t>(sg.g) |
                         reinterpret_cast<uintptr_t>(sg.m) | reinterpret_cast<uintptr_t>(sg.v);
    sg.vec = (cnt[k] % 4 == 0 && (al & 15) == 0) ? 1u : 0u;
    const uint64_t units = sg.vec ? cnt[k] / 4 : cnt[k];
    most = units > most ? units : most;
    off += padded(cnt[k]);
  }
  a.seg[4].lr_alt = cfg->lr_sh_rest;
  a.seg[4].period = (uint32_t)K3;
  a.seg[1].penalty = (float)((double)cfg->size_penalty / (double)n);
  a.b1 = cfg->beta1;
  a.b2 = cfg->beta2;
  a.eps = cfg->eps;
  a.step_scale = (float)(1.0 / (1.0 - std::pow((double)cfg->beta1, (double)step)));
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)cfg->beta2, (double)step)));
  const uint64_t want = (most + kAdamThreads - 1) / kAdamThreads;
  const unsigned bx = (unsigned)(want < (uint64_t)kAdamBlocks ? want : (uint64_t)kAdamBlocks);
  hipStream_t s = (hipStream_t)stream;
  {
    TimedScope ts("adam", s);
    hipLaunchKernelGGL(k_adam, dim3(bx, kAdamGroups), dim3(kAdamThreads), 0, s, a);
  }
  return check_launch("gs_adam_step");
}
