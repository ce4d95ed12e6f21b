// The fp32 projection of one Gaussian, shared by k-project (which writes its outputs) and k-pbwd
// (which replays it to take exactly the forward's decisions: culling, the J clamps, the det
// clamp). Definitions: "Gaussian splatting in PyTorch", sections 1 (activations), 2
// (Sigma = R S S^T R^T), 3 (world->camera, EWA Jacobian with the clamp widened by 0.3
// tan(half-FoV)) and 4 (eps2d dilation, conic, gsplat's per-axis radius with the opacity-aware
// extent min(3.33, sqrt(2 ln(255 o))), and the section's two variants as camera options: the
// 3DGS radius ceil(3 sqrt(lambda_max)) on both axes, and the antialiased opacity o times
// sqrt(det Sigma2d / det Sigma') with Sigma2d the covariance before the dilation, on which the
// cull and the extent then act). Every expression is evaluated in fp32 in a fixed order with no
// contraction, so radii, rectangles and tile counts are reproducible bit for bit.
#pragma once

#include "gs_internal.h"

namespace gs {

// Real spherical harmonics scaled so that B_00 = 1 (textbook basis, order m = -l..l, no
// Condon-Shortley phase). d = (x, y, z) is a unit vector.
__device__ __forceinline__ void sh_basis_f32(int degree, float x, float y, float z, float* B) {
  // sqrt(3), sqrt(15), sqrt(5)/2, sqrt(15)/2, sqrt(35/8), sqrt(105), sqrt(21/8), sqrt(7)/2,
  // sqrt(105)/2, each rounded to the nearest float
  const float s3 = 0x1.bb67aep+0f, s15 = 0x1.efbdecp+1f, s5h = 0x1.1e377ap+0f, s15h = 0x1.efbdecp+0f,
              s358 = 0x1.0bbb30p+1f, s105 = 0x1.47e706p+3f, s218 = 0x1.9ec474p+0f, s7h = 0x1.52a7fap+0f,
              s105h = 0x1.47e706p+2f;
  B[0] = 1.0f;
  if (degree < 1) return;
  B[1] = s3 * y;
  B[2] = s3 * z;
  B[3] = s3 * x;
  if (degree < 2) return;
  B[4] = s15 * x * y;
  B[5] = s15 * y * z;
  B[6] = s5h * (3.0f * z * z - 1.0f);
  B[7] = s15 * x * z;
  B[8] = s15h * (x * x - y * y);
  if (degree < 3) return;
  B[9] = s358 * y * (3.0f * x * x - y * y);
  B[10] = s105 * x * y * z;
  B[11] = s218 * y * (5.0f * z * z - 1.0f);
  B[12] = s7h * z * (5.0f * z * z - 3.0f);
  B[13] = s218 * x * (5.0f * z * z - 1.0f);
  B[14] = s105h * z * (x * x - y * y);
  B[15] = s358 * x * (x * x - 3.0f * y * y);
}

__device__ __forceinline__ bool fin(float x) { return __builtin_isfinite(x); }

struct ProjF32 {
  bool defined;  // passed the near plane and every finiteness test
  bool drawn;    // defined, o >= 1/255 and at least one tile on screen
  bool clamp_x, clamp_y, det_clamped;
  float m2d[2], con[3], depth, o, col[3];  // o: the opacity the blend uses (o_act comp)
  float o_act, comp;                        // sigmoid(logit) and the antialiased factor (1 if off)
  int32_t rad[2];
  uint32_t tiles;
};

// shc: the Gaussian's (DEG+1)^2 x 3 SH coefficients (only read when WITH_COLOR)
// Tight counts of rectangles taller than this many rows are left to the projection kernel's
// wave (one lane per row) so that one tall splat does not hold up the lanes of its wave.
constexpr uint32_t kTightLaneRows = 16;
constexpr uint32_t kTightPending = 0xFFFFFFFFu;

template <int DEG, bool WITH_COLOR>
__device__ __forceinline__ ProjF32 project_f32(float m0, float m1, float m2, float l0, float l1, float l2, float4 q4,
                                               float logit, const float* shc, const DevCamera& cam) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  ProjF32 P;
  P.defined = P.drawn = P.clamp_x = P.clamp_y = P.det_clamped = false;
  P.m2d[0] = P.m2d[1] = 0.0f;
  P.con[0] = P.con[1] = P.con[2] = 0.0f;
  P.depth = P.o = P.o_act = 0.0f;
  P.comp = 1.0f;
  P.col[0] = P.col[1] = P.col[2] = 0.0f;
  P.rad[0] = P.rad[1] = 0;
  P.tiles = 0;

  bool ok = fin(m0) && fin(m1) && fin(m2) && fin(l0) && fin(l1) && fin(l2) && fin(q4.x) && fin(q4.y) &&
            fin(q4.z) && fin(q4.w) && fin(logit);
#pragma unroll
  for (int i = 0; i < K * 3; ++i) ok = ok && fin(shc[i]);
  if (!ok) return P;

  // section 1: activations
  const float qn = omax(sqrtf(((q4.x * q4.x + q4.y * q4.y) + q4.z * q4.z) + q4.w * q4.w), 1e-12f);
  const float w = q4.x / qn, x = q4.y / qn, y = q4.z / qn, z = q4.w / qn;
  const float s[3] = {act_exp(l0), act_exp(l1), act_exp(l2)};
  const float o = 1.0f / (1.0f + act_exp(-logit));

  // section 2: R(q), M = R diag(s), Sigma = M M^T
  float R[9];
  R[0] = 1.0f - 2.0f * (y * y + z * z);
  R[1] = 2.0f * (x * y - w * z);
  R[2] = 2.0f * (x * z + w * y);
  R[3] = 2.0f * (x * y + w * z);
  R[4] = 1.0f - 2.0f * (x * x + z * z);
  R[5] = 2.0f * (y * z - w * x);
  R[6] = 2.0f * (x * z - w * y);
  R[7] = 2.0f * (y * z + w * x);
  R[8] = 1.0f - 2.0f * (x * x + y * y);
  float M[9], Sig[9];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) M[i * 3 + j] = R[i * 3 + j] * s[j];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      Sig[i * 3 + j] = (M[i * 3 + 0] * M[j * 3 + 0] + M[i * 3 + 1] * M[j * 3 + 1]) + M[i * 3 + 2] * M[j * 3 + 2];

  // section 3: t = W mean + w0, Sigma_c = W Sigma W^T
  const float* V = cam.V;
  float t[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) t[r] = ((V[r * 4 + 0] * m0 + V[r * 4 + 1] * m1) + V[r * 4 + 2] * m2) + V[r * 4 + 3];
  float WS[9], Sc[9];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      WS[i * 3 + j] = (V[i * 4 + 0] * Sig[0 * 3 + j] + V[i * 4 + 1] * Sig[1 * 3 + j]) + V[i * 4 + 2] * Sig[2 * 3 + j];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      Sc[i * 3 + j] = (WS[i * 3 + 0] * V[j * 4 + 0] + WS[i * 3 + 1] * V[j * 4 + 1]) + WS[i * 3 + 2] * V[j * 4 + 2];
  const float tx = t[0], ty = t[1], tz = t[2];
  if (!(tz > cam.near_plane)) return P;

  // EWA Jacobian with x/z, y/z clamped to the widened view (the 2D mean is not clamped)
  const float fx = cam.fx, fy = cam.fy, cx = cam.cx, cy = cam.cy;
  const float tan_fovx = 0.5f * (float)cam.W / fx, tan_fovy = 0.5f * (float)cam.H / fy;
  const float lxl = -(cx / fx + 0.3f * tan_fovx), lxh = ((float)cam.W - cx) / fx + 0.3f * tan_fovx;
  const float lyl = -(cy / fy + 0.3f * tan_fovy), lyh = ((float)cam.H - cy) / fy + 0.3f * tan_fovy;
  const float xz = tx / tz, yz = ty / tz;
  P.clamp_x = (xz < lxl) || (xz > lxh);
  P.clamp_y = (yz < lyl) || (yz > lyh);
  const float jx = tz * omin(omax(xz, lxl), lxh);
  const float jy = tz * omin(omax(yz, lyl), lyh);
  const float J[6] = {fx / tz, 0.0f, -fx * jx / (tz * tz), 0.0f, fy / tz, -fy * jy / (tz * tz)};

  // section 4: Sigma' = J Sigma_c J^T + 0.3 I, conic, mean2d
  float JS[6];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      JS[i * 3 + j] = (J[i * 3 + 0] * Sc[0 * 3 + j] + J[i * 3 + 1] * Sc[1 * 3 + j]) + J[i * 3 + 2] * Sc[2 * 3 + j];
  const float c00 = (JS[0] * J[0] + JS[1] * J[1]) + JS[2] * J[2];
  const float c01 = (JS[0] * J[3] + JS[1] * J[4]) + JS[2] * J[5];
  const float c11 = (JS[3] * J[3] + JS[4] * J[4]) + JS[5] * J[5];
  const float a = c00 + 0.3f, b = c01, c = c11 + 0.3f;
  const float det_raw = a * c - b * b;
  P.det_clamped = det_raw < 1e-10f;
  const float det = omax(det_raw, 1e-10f);
  const float con0 = c / det, con1 = -b / det, con2 = a / det;
  // antialiased: o sqrt(det Sigma2d / det Sigma'), which keeps o 2 pi sqrt(det) of the undilated
  // Gaussian
  const float det0 = c00 * c11 - c01 * c01;
  const float comp = cam.antialiased ? sqrtf(omax(det0, 0.0f) / det) : 1.0f;
  const float o_eff = cam.antialiased ? o * comp : o;
  const float mx = fx * tx / tz + cx, my = fy * ty / tz + cy;
  if (!(fin(a) && fin(b) && fin(c) && fin(con0) && fin(con1) && fin(con2) && fin(mx) && fin(my))) return P;

  // colour: sum_lm k_lm B_lm(d), d = unit direction from the camera centre to the mean
  if (WITH_COLOR) {
    if (DEG == 0) {
      P.col[0] = shc[0]; P.col[1] = shc[1]; P.col[2] = shc[2];
    } else {
      float C[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) C[j] = -((V[0 * 4 + j] * V[3] + V[1 * 4 + j] * V[7]) + V[2 * 4 + j] * V[11]);
      const float d0 = m0 - C[0], d1 = m1 - C[1], d2 = m2 - C[2];
      const float dn = omax(sqrtf((d0 * d0 + d1 * d1) + d2 * d2), 1e-12f);
      float B[16];
      sh_basis_f32(DEG, d0 / dn, d1 / dn, d2 / dn, B);
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) {
        float acc = 0.0f;
#pragma unroll
        for (int l = 0; l < K; ++l) acc = acc + shc[l * 3 + ch] * B[l];
        P.col[ch] = acc;
      }
    }
  }
  P.m2d[0] = mx; P.m2d[1] = my;
  P.con[0] = con0; P.con[1] = con1; P.con[2] = con2;
  P.depth = tz;
  P.o = o_eff;
  P.o_act = o;
  P.comp = comp;
  P.defined = true;

  // radius: opacity-aware per-axis extent (or the 3DGS radius); nothing drawn below 1/255
  if (o_eff < 1.0f / 255.0f) return P;
  float rx, ry;
  if (cam.radius_mode == 1) {
    const float mid = 0.5f * (a + c);
    const float lam = mid + sqrtf(omax(mid * mid - det, 0.1f));
    rx = ry = omin(ceilf(3.0f * sqrtf(lam)), 16777216.0f);
  } else {
    float kk = 2.0f * act_log(255.0f * o_eff);
    if (!(kk > 0.0f)) kk = 0.0f;
    float k = sqrtf(kk);
    if (k > 3.33f) k = 3.33f;
    rx = omin(ceilf(k * sqrtf(a)), 16777216.0f);
    ry = omin(ceilf(k * sqrtf(c)), 16777216.0f);
  }
  const TileRect rc = tile_rect(mx, my, rx, ry, cam.tiles_x, cam.tiles_y);
  if (!(rc.x1 > rc.x0 && rc.y1 > rc.y0)) return P;
  uint32_t tiles = (uint32_t)((rc.x1 - rc.x0) * (rc.y1 - rc.y0));
  if (cam.tight_tiles) {  // only the tiles of the rectangle the ellipse reaches
    if (WITH_COLOR && rc.y1 - rc.y0 > (int)kTightLaneRows) {
      tiles = kTightPending;  // counted by the whole wave (k_project), which also undraws a 0
    } else {
      const TightShape ts = tight_shape(mx, my, con0, con1, con2, o_eff);
      tiles = 0;
      for (int ty = rc.y0; ty < rc.y1; ++ty) {
        const int2 sp = tight_row(ts, ty, rc.x0, rc.x1);
        tiles += (uint32_t)(sp.y - sp.x);
      }
      if (tiles == 0) return P;
    }
  }
  P.rad[0] = (int32_t)rx;
  P.rad[1] = (int32_t)ry;
  P.tiles = tiles;
  P.drawn = true;
  return P;
}

}  // namespace gs
