// k-project: one thread per Gaussian -- activations, covariance, EWA projection, culling,
// conic, opacity-aware radius, tile rectangle/count and SH colour.
//
// Definitions: "Gaussian splatting in PyTorch", sections 1 (activations), 2 (Sigma = R S S^T
// R^T), 3 (world->camera, EWA Jacobian with the clamp widened by 0.3 tan(half-FoV)) and 4 (eps2d
// dilation, conic, gsplat's per-axis radius with the opacity-aware extent
// min(3.33, sqrt(2 ln(255 o)))). Every expression is evaluated in fp32 in a fixed order with no
// contraction, so radii, rectangles and tile counts are reproducible bit for bit.
//
// The work is O(N) with ~60 B read (SH degree 0; 236 B at degree 3) and 52 B written per
// Gaussian: HBM-bound and a few microseconds even at 742k Gaussians. Loads are per-thread
// contiguous records; consecutive threads read consecutive records, so each wave's reads cover
// whole cache lines.
#include "project_core.h"

namespace gs {
namespace {

constexpr int kProjectThreads = 256;

template <int DEG>
__global__ __launch_bounds__(kProjectThreads) void k_project(
    int32_t n, const float* __restrict__ means, const float* __restrict__ log_scales,
    const float* __restrict__ quats, const float* __restrict__ logits, const float* __restrict__ sh,
    DevCamera cam, float* __restrict__ means2d, float* __restrict__ conics, float* __restrict__ depths,
    float* __restrict__ opacities, float* __restrict__ colors, int32_t* __restrict__ radii,
    uint32_t* __restrict__ tiles_touched) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int g = blockIdx.x * kProjectThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  if (blockIdx.x * kProjectThreads + (threadIdx.x & ~63) >= n) return;  // whole waves past n only
  const bool valid = g < n;
  const int gg = valid ? g : n - 1;  // lanes past n compute a copy of the last Gaussian, store nothing
  float shc[K * 3];
#pragma unroll
  for (int i = 0; i < K * 3; ++i) shc[i] = sh[(size_t)gg * (K * 3) + i];
  ProjF32 P = project_f32<DEG, true>(means[3 * gg], means[3 * gg + 1], means[3 * gg + 2], log_scales[3 * gg],
                                      log_scales[3 * gg + 1], log_scales[3 * gg + 2],
                                      *reinterpret_cast<const float4*>(quats + 4 * gg), logits[gg], shc, cam);
  if (cam.tight_tiles) {
    // tight counts of tall rectangles: the wave takes them one at a time, one lane per row, and
    // adds the rows' tiles (integers: the order does not matter)
    uint64_t pend = __ballot(valid && P.drawn && P.tiles == kTightPending);
    while (pend) {
      const int src = __builtin_ctzll(pend);
      pend &= pend - 1;
      auto bf = [&](float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src)); };
      const float mx = bf(P.m2d[0]), my = bf(P.m2d[1]);
      const float rx = (float)__builtin_amdgcn_readlane(P.rad[0], src);
      const float ry = (float)__builtin_amdgcn_readlane(P.rad[1], src);
      const TileRect rc = tile_rect(mx, my, rx, ry, cam.tiles_x, cam.tiles_y);
      const TightShape ts = tight_shape(mx, my, bf(P.con[0]), bf(P.con[1]), bf(P.con[2]), bf(P.o));
      uint32_t cnt = 0;
      for (int ty = rc.y0 + lane; ty < rc.y1; ty += 64) {
        const int2 sp = tight_row(ts, ty, rc.x0, rc.x1);
        cnt += (uint32_t)(sp.y - sp.x);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) cnt += (uint32_t)__shfl_xor((int)cnt, off, 64);
      if (lane == src) {
        P.tiles = cnt;
        if (cnt == 0) {  // the ellipse reaches no pixel centre: not drawn
          P.drawn = false;
          P.rad[0] = P.rad[1] = 0;
        }
      }
    }
  }
  if (!valid) return;
  means2d[2 * g] = P.m2d[0];
  means2d[2 * g + 1] = P.m2d[1];
  conics[3 * g] = P.con[0];
  conics[3 * g + 1] = P.con[1];
  conics[3 * g + 2] = P.con[2];
  depths[g] = P.depth;
  opacities[g] = P.o;
  colors[3 * g] = P.col[0];
  colors[3 * g + 1] = P.col[1];
  colors[3 * g + 2] = P.col[2];
  radii[2 * g] = P.rad[0];
  radii[2 * g + 1] = P.rad[1];
  tiles_touched[g] = P.tiles;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" gs_status gs_project(int32_t n, int32_t sh_degree, const float* d_means, const float* d_log_scales,
                                const float* d_quats, const float* d_opacity_logits, const float* d_sh,
                                const gs_camera* cam, const gs_projected* out, void* stream) {
  std::string why;
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, "gs_project: n < 0");
  if (sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return set_error(GS_ERR_INVALID_ARG, "gs_project: sh_degree not in 0..3");
  if (!valid_camera(cam, &why)) return set_error(GS_ERR_INVALID_ARG, "gs_project: " + why);
  if (!out) return set_error(GS_ERR_INVALID_ARG, "gs_project: out is NULL");
  if (n == 0) return GS_OK;
  if (!d_means || !d_log_scales || !d_quats || !d_opacity_logits || !d_sh || !out->d_means2d || !out->d_conics ||
      !out->d_depths || !out->d_opacities || !out->d_colors || !out->d_radii || !out->d_tiles_touched)
    return set_error(GS_ERR_INVALID_ARG, "gs_project: NULL pointer with n > 0");
  if ((reinterpret_cast<uintptr_t>(d_quats) & 15) != 0)
    return set_error(GS_ERR_INVALID_ARG, "gs_project: d_quats must be 16-byte aligned");
  const DevCamera dc = to_dev(*cam);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((n + kProjectThreads - 1) / kProjectThreads), block(kProjectThreads);
  {
    TimedScope ts("project", s);
#define GS_LAUNCH_PROJECT(D)                                                                               \
  hipLaunchKernelGGL(k_project<D>, grid, block, 0, s, n, d_means, d_log_scales, d_quats, d_opacity_logits, d_sh, \
                     dc, out->d_means2d, out->d_conics, out->d_depths, out->d_opacities, out->d_colors,        \
                     out->d_radii, out->d_tiles_touched)
    switch (sh_degree) {
      case 0: GS_LAUNCH_PROJECT(0); break;
      case 1: GS_LAUNCH_PROJECT(1); break;
      case 2: GS_LAUNCH_PROJECT(2); break;
      default: GS_LAUNCH_PROJECT(3); break;
    }
#undef GS_LAUNCH_PROJECT
  }
  return check_launch("gs_project");
}
