// L1 photometric loss and its gradient: the L1 term of section 7's training loss
// ((1 - lambda) L1 + lambda (1 - SSIM)) in "Gaussian splatting in PyTorch".
// L = mean |image - target| over h*w*3 values; dL/dimage = sign(image - target) / (3 h w).
// Elementwise and HBM-bound (8 B read + 4 B written per value); float4 vectorised when all three
// arrays are 16-byte aligned, scalar otherwise. The loss
// value, when asked for, is reduced per workgroup and added atomically into *loss (cleared first,
// in stream order), so its last bits may vary run to run.
#include <cmath>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kLossThreads = 256;
constexpr int kLossBlocks = 1024;

__device__ __forceinline__ float sgn(float d) { return d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f); }

template <bool VEC>
__global__ __launch_bounds__(kLossThreads) void k_l1(size_t count, const float* __restrict__ img,
                                                     const float* __restrict__ tgt, float* __restrict__ grad,
                                                     float inv_count, float* __restrict__ loss) {
  __shared__ float s_red[kLossThreads / 64];
  float acc = 0.0f;
  const size_t n4 = VEC ? count / 4 : 0;
  const size_t stride = (size_t)gridDim.x * kLossThreads;
  for (size_t i = blockIdx.x * (size_t)kLossThreads + threadIdx.x; i < n4; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(img)[i];
    const float4 b = reinterpret_cast<const float4*>(tgt)[i];
    const float4 d = make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
    reinterpret_cast<float4*>(grad)[i] =
        make_float4(sgn(d.x) * inv_count, sgn(d.y) * inv_count, sgn(d.z) * inv_count, sgn(d.w) * inv_count);
    acc += (fabsf(d.x) + fabsf(d.y)) + (fabsf(d.z) + fabsf(d.w));
  }
  for (size_t i = n4 * 4 + blockIdx.x * (size_t)kLossThreads + threadIdx.x; i < count; i += stride) {
    const float d = img[i] - tgt[i];
    grad[i] = sgn(d) * inv_count;
    acc += fabsf(d);
  }
  if (!loss) return;
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) unsafeAtomicAdd(loss, ((s_red[0] + s_red[1]) + (s_red[2] + s_red[3])) * inv_count);
}

__global__ void k_zero_one(float* __restrict__ p) { *p = 0.0f; }

// ---------------------------------------------------------------------------------------------
// L1 + SSIM: L = (1 - lam) L1 + lam (1 - SSIM), the full training loss of section 7, with SSIM of
// Wang et al. 2004: per channel, local means and (co)variances under an 11 x 11 Gaussian window
// (sigma 1.5, normalised, the image padded with zeros), C1 = 0.01^2, C2 = 0.03^2,
//   S = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy + C2)),
// SSIM = the mean of S over the h w 3 values. Its gradient goes through the window statistics:
// with e_xx = w * x^2 and e_xy = w * (x y), the sum over the map of dS/dx at q is
//   (w * dS/dmu_x)(q) + 2 x_q (w * dS/de_xx)(q) + y_q (w * dS/de_xy)(q)
// (the zero-padded filter's adjoint is the same symmetric window, zero padded).
// Two launches over 16 x 16 output tiles, each staging a 26 x 26 input region (5-pixel halo) in
// LDS and filtering it separably (a horizontal pass into LDS, then a vertical one):
//   k_ssim_stats: the five window statistics of each channel, S, and the three partials of S
//     per pixel and channel, written as nine planes; per-tile sums of S and |x - y|;
//   k_ssim_grad:  the three partial planes filtered again, and dL/dx; workgroup 0 adds the
//     per-tile sums in a fixed order (in double) into the loss value.
// ---------------------------------------------------------------------------------------------
constexpr int kSsimTile = 16, kSsimHalo = 5, kSsimIn = kSsimTile + 2 * kSsimHalo, kSsimTaps = 2 * kSsimHalo + 1;

struct SsimArgs {
  float g[kSsimTaps];  // the normalised 1D window
  int32_t W, H;
  float lam, inv_n;    // lambda and 1 / (3 h w)
  float c1, c2;
};

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Horizontal pass shared by both kernels: thread t < 208 filters row t / 8 of the 26-row region
// at output columns 2 (t % 8) and 2 (t % 8) + 1, reading the 12 inputs both need once.
constexpr int kSsimHThreads = kSsimIn * (kSsimTile / 2);  // 208

__global__ __launch_bounds__(kSsimTile * kSsimTile) void k_ssim_stats(const float* __restrict__ img,
                                                                       const float* __restrict__ tgt, SsimArgs a,
                                                                       float* __restrict__ part,
                                                                       float2* __restrict__ tile_sums) {
  __shared__ float s_x[3][kSsimIn][kSsimIn];
  __shared__ float s_y[3][kSsimIn][kSsimIn];
  __shared__ float s_h[1][5][kSsimIn][kSsimTile];
  __shared__ float s_red[2][4];
  const int tid = threadIdx.x, lx = tid & 15, ly = tid >> 4;
  const int ox = blockIdx.x * kSsimTile - kSsimHalo, oy = blockIdx.y * kSsimTile - kSsimHalo;
  // the 26 x 26 RGB region, zero outside the image: a region row is 78 consecutive floats, read
  // by threads 0..233 (three rows at a time), each keeping its channel and column
  // (every load is issued before the first LDS store, so the latencies overlap)
  if (tid < 3 * kSsimIn * 3) {
    const int q = tid % (kSsimIn * 3), r0 = tid / (kSsimIn * 3), ch = q % 3, col = q / 3;
    const int gx = ox + col;
    constexpr int kRows = (kSsimIn + 2) / 3;  // 9
    float vx[kRows], vy[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = r0 + 3 * i, gy = oy + r;
      const bool in = r < kSsimIn && gx >= 0 && gx < a.W && gy >= 0 && gy < a.H;
      const size_t src = ((size_t)gy * a.W + gx) * 3 + ch;
      vx[i] = in ? img[src] : 0.0f;
      vy[i] = in ? tgt[src] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = r0 + 3 * i;
      if (r < kSsimIn) {
        s_x[ch][r][col] = vx[i];
        s_y[ch][r][col] = vy[i];
      }
    }
  }
  __syncthreads();
  const int px = blockIdx.x * kSsimTile + lx, py = blockIdx.y * kSsimTile + ly;
  const bool inside = px < a.W && py < a.H;
  const size_t plane = (size_t)a.W * a.H, pix = (size_t)py * a.W + px;
  float ssum = 0.0f, l1sum = 0.0f;
  for (int ch = 0; ch < 3; ++ch) {
    if (tid < kSsimHThreads) {
      const int r = tid >> 3, c0 = (tid & 7) * 2;
      // the 12 inputs and their products, formed once for both outputs
      float xv[kSsimTaps + 1], yv[kSsimTaps + 1], xx[kSsimTaps + 1], yy[kSsimTaps + 1], xy[kSsimTaps + 1];
#pragma unroll
      for (int k = 0; k <= kSsimTaps; ++k) {
        xv[k] = s_x[ch][r][c0 + k];
        yv[k] = s_y[ch][r][c0 + k];
        xx[k] = xv[k] * xv[k];
        yy[k] = yv[k] * yv[k];
        xy[k] = xv[k] * yv[k];
      }
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        float m1 = 0.0f, m2 = 0.0f, e11 = 0.0f, e22 = 0.0f, e12 = 0.0f;
#pragma unroll
        for (int k = 0; k < kSsimTaps; ++k) {
          const float w = a.g[k];
          m1 = fmaf(w, xv[o + k], m1);
          m2 = fmaf(w, yv[o + k], m2);
          e11 = fmaf(w, xx[o + k], e11);
          e22 = fmaf(w, yy[o + k], e22);
          e12 = fmaf(w, xy[o + k], e12);
        }
        float(*h)[kSsimIn][kSsimTile] = s_h[0];
        h[0][r][c0 + o] = m1;
        h[1][r][c0 + o] = m2;
        h[2][r][c0 + o] = e11;
        h[3][r][c0 + o] = e22;
        h[4][r][c0 + o] = e12;
      }
    }
    __syncthreads();
    float mx = 0.0f, my = 0.0f, exx = 0.0f, eyy = 0.0f, exy = 0.0f;
    const float(*h)[kSsimIn][kSsimTile] = s_h[0];
#pragma unroll
    for (int k = 0; k < kSsimTaps; ++k) {
      const float w = a.g[k];
      mx = fmaf(w, h[0][ly + k][lx], mx);
      my = fmaf(w, h[1][ly + k][lx], my);
      exx = fmaf(w, h[2][ly + k][lx], exx);
      eyy = fmaf(w, h[3][ly + k][lx], eyy);
      exy = fmaf(w, h[4][ly + k][lx], exy);
    }
    if (inside) {
      const float sxx = exx - mx * mx, syy = eyy - my * my, sxy = exy - mx * my;
      const float A1 = 2.0f * mx * my + a.c1, A2 = 2.0f * sxy + a.c2;
      const float B1 = (mx * mx + my * my) + a.c1, B2 = (sxx + syy) + a.c2;
      const float iA1 = rcp(A1), iA2 = rcp(A2), iB1 = rcp(B1), iB2 = rcp(B2);
      const float S = (A1 * A2) * (iB1 * iB2);
      const float d_mx = S * ((2.0f * my * iA1 - 2.0f * mx * iB1) + (2.0f * mx * iB2 - 2.0f * my * iA2));
      part[(size_t)(ch * 3 + 0) * plane + pix] = d_mx;
      part[(size_t)(ch * 3 + 1) * plane + pix] = -S * iB2;
      part[(size_t)(ch * 3 + 2) * plane + pix] = 2.0f * S * iA2;
      ssum += S;
      l1sum += fabsf(s_x[ch][ly + kSsimHalo][lx + kSsimHalo] - s_y[ch][ly + kSsimHalo][lx + kSsimHalo]);
    }
    __syncthreads();  // s_h is rewritten for the next channel
  }
  for (int off = 32; off > 0; off >>= 1) {
    ssum += __shfl_down(ssum, off, 64);
    l1sum += __shfl_down(l1sum, off, 64);
  }
  if ((tid & 63) == 0) {
    s_red[0][tid >> 6] = ssum;
    s_red[1][tid >> 6] = l1sum;
  }
  __syncthreads();
  if (tid == 0)
    tile_sums[blockIdx.y * gridDim.x + blockIdx.x] =
        make_float2((s_red[0][0] + s_red[0][1]) + (s_red[0][2] + s_red[0][3]),
                    (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]));
}

__global__ __launch_bounds__(kSsimTile * kSsimTile) void k_ssim_grad(const float* __restrict__ img,
                                                                      const float* __restrict__ tgt, SsimArgs a,
                                                                      const float* __restrict__ part,
                                                                      const float2* __restrict__ tile_sums,
                                                                      int32_t ntiles, float* __restrict__ grad,
                                                                      float* __restrict__ loss) {
  __shared__ float s_p[9][kSsimIn][kSsimIn];
  __shared__ float s_h[2][3][kSsimIn][kSsimTile];  // two buffers: channel c uses c & 1
  const int tid = threadIdx.x, lx = tid & 15, ly = tid >> 4;
  const int ox = blockIdx.x * kSsimTile - kSsimHalo, oy = blockIdx.y * kSsimTile - kSsimHalo;
  const int px = blockIdx.x * kSsimTile + lx, py = blockIdx.y * kSsimTile + ly;
  const bool inside = px < a.W && py < a.H;
  const size_t plane = (size_t)a.W * a.H, pix = (size_t)py * a.W + px;
  // region loads: threads 0..233, nine rows at a time, each keeping its column
  const int lq = tid % kSsimIn, lr0 = tid / kSsimIn;
  const int gx = ox + lq;
  // the nine partial planes' regions: all loads in flight before the first LDS store
  if (tid < 9 * kSsimIn) {
    constexpr int kRows = (kSsimIn + 8) / 9;  // 3
    float v[kRows][9];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = lr0 + 9 * i, gy = oy + r;
      const bool in = r < kSsimIn && gx >= 0 && gx < a.W && gy >= 0 && gy < a.H;
      const size_t src = (size_t)gy * a.W + gx;
#pragma unroll
      for (int m = 0; m < 9; ++m) v[i][m] = in ? part[(size_t)m * plane + src] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = lr0 + 9 * i;
      if (r < kSsimIn) {
#pragma unroll
        for (int m = 0; m < 9; ++m) s_p[m][r][lq] = v[i][m];
      }
    }
  }
  __syncthreads();
  for (int ch = 0; ch < 3; ++ch) {
    float(*h)[kSsimIn][kSsimTile] = s_h[ch & 1];
    if (tid < kSsimHThreads) {
      const int r = tid >> 3, c0 = (tid & 7) * 2;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float v[kSsimTaps + 1];
#pragma unroll
        for (int k = 0; k <= kSsimTaps; ++k) v[k] = s_p[ch * 3 + m][r][c0 + k];
        float f0 = 0.0f, f1 = 0.0f;
#pragma unroll
        for (int k = 0; k < kSsimTaps; ++k) {
          f0 = fmaf(a.g[k], v[k], f0);
          f1 = fmaf(a.g[k], v[k + 1], f1);
        }
        h[m][r][c0] = f0;
        h[m][r][c0 + 1] = f1;
      }
    }
    __syncthreads();
    float F0 = 0.0f, F1 = 0.0f, F2 = 0.0f;
#pragma unroll
    for (int k = 0; k < kSsimTaps; ++k) {
      const float w = a.g[k];
      F0 = fmaf(w, h[0][ly + k][lx], F0);
      F1 = fmaf(w, h[1][ly + k][lx], F1);
      F2 = fmaf(w, h[2][ly + k][lx], F2);
    }
    if (inside) {
      const float x = img[pix * 3 + ch], y = tgt[pix * 3 + ch];
      const float dS = fmaf(2.0f * x, F1, fmaf(y, F2, F0));
      grad[pix * 3 + ch] = ((1.0f - a.lam) * sgn(x - y) - a.lam * dS) * a.inv_n;
    }
    // no barrier: the next channel writes the other s_h buffer (see k_ssim_stats)
  }
  if (loss && blockIdx.x == 0 && blockIdx.y == 0) {
    // the per-tile sums in a fixed order: thread t takes tiles t, t + 256, ..., then a fixed tree
    __shared__ double s_d[2][kSsimTile * kSsimTile];
    double ss = 0.0, l1 = 0.0;
    for (int t = tid; t < ntiles; t += kSsimTile * kSsimTile) {
      ss += (double)tile_sums[t].x;
      l1 += (double)tile_sums[t].y;
    }
    s_d[0][tid] = ss;
    s_d[1][tid] = l1;
    __syncthreads();
    for (int half = kSsimTile * kSsimTile / 2; half > 0; half >>= 1) {
      if (tid < half) {
        s_d[0][tid] += s_d[0][tid + half];
        s_d[1][tid] += s_d[1][tid + half];
      }
      __syncthreads();
    }
    if (tid == 0) {
      const double n = 3.0 * (double)a.W * (double)a.H;
      *loss = (float)((1.0 - (double)a.lam) * s_d[1][0] / n + (double)a.lam * (1.0 - s_d[0][0] / n));
    }
  }
}

}  // namespace
}  // namespace gs

using namespace gs;

namespace {
size_t ssim_tiles(int32_t w, int32_t h) {
  return (size_t)((w + kSsimTile - 1) / kSsimTile) * (size_t)((h + kSsimTile - 1) / kSsimTile);
}
size_t ssim_part_bytes(int32_t w, int32_t h) { return align_up((size_t)w * h * 9 * 4, 256); }
}  // namespace

extern "C" gs_status gs_loss_l1(int32_t width, int32_t height, const float* d_image, const float* d_target,
                                float* d_dL_dimage, float* d_loss, void* stream) {
  if (width <= 0 || height <= 0) return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1: width/height <= 0");
  if (!d_image || !d_target || !d_dL_dimage) return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1: NULL pointer");
  const uintptr_t align = reinterpret_cast<uintptr_t>(d_image) | reinterpret_cast<uintptr_t>(d_target) |
                          reinterpret_cast<uintptr_t>(d_dL_dimage);
  if ((align & 3) != 0) return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1: arrays must be 4-byte aligned");
  const bool vec = (align & 15) == 0;
  const size_t count = (size_t)width * height * 3;
  hipStream_t s = (hipStream_t)stream;
  const size_t want = ((vec ? count / 4 : count) + kLossThreads - 1) / kLossThreads;
  const int blocks = (int)(want < (size_t)kLossBlocks ? (want > 0 ? want : 1) : kLossBlocks);
  {
    TimedScope ts("loss_l1", s);
    if (d_loss) hipLaunchKernelGGL(k_zero_one, dim3(1), dim3(1), 0, s, d_loss);
    if (vec)
      hipLaunchKernelGGL(k_l1<true>, dim3(blocks), dim3(kLossThreads), 0, s, count, d_image, d_target, d_dL_dimage,
                         1.0f / (float)count, d_loss);
    else
      hipLaunchKernelGGL(k_l1<false>, dim3(blocks), dim3(kLossThreads), 0, s, count, d_image, d_target, d_dL_dimage,
                         1.0f / (float)count, d_loss);
  }
  return check_launch("gs_loss_l1");
}

extern "C" size_t gs_loss_ssim_workspace_bytes(int32_t width, int32_t height) {
  if (width <= 0 || height <= 0) return 0;
  return ssim_part_bytes(width, height) + align_up(ssim_tiles(width, height) * sizeof(float2), 256);
}

extern "C" gs_status gs_loss_l1_ssim(int32_t width, int32_t height, const float* d_image, const float* d_target,
                                     float lambda, void* d_workspace, size_t workspace_bytes, float* d_dL_dimage,
                                     float* d_loss, void* stream) {
  if (width <= 0 || height <= 0) return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1_ssim: width/height <= 0");
  if ((int64_t)width * height * 9 >= ((int64_t)1 << 31))
    return set_error(GS_ERR_LIMIT, "gs_loss_l1_ssim: image too large");
  if (!d_image || !d_target || !d_dL_dimage || !d_workspace)
    return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1_ssim: NULL pointer");
  if (!(lambda >= 0.0f && lambda <= 1.0f)) return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1_ssim: lambda not in [0, 1]");
  if (workspace_bytes < gs_loss_ssim_workspace_bytes(width, height))
    return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1_ssim: workspace smaller than gs_loss_ssim_workspace_bytes()");
  if ((reinterpret_cast<uintptr_t>(d_workspace) & 255) != 0)
    return set_error(GS_ERR_INVALID_ARG, "gs_loss_l1_ssim: workspace must be 256-byte aligned");
  SsimArgs a{};
  double g[kSsimTaps], sum = 0.0;
  for (int k = 0; k < kSsimTaps; ++k) {
    const double r = (double)(k - kSsimHalo);
    g[k] = std::exp(-r * r / (2.0 * 1.5 * 1.5));
    sum += g[k];
  }
  for (int k = 0; k < kSsimTaps; ++k) a.g[k] = (float)(g[k] / sum);
  a.W = width;
  a.H = height;
  a.lam = lambda;
  a.inv_n = (float)(1.0 / (3.0 * (double)width * (double)height));
  a.c1 = 0.01f * 0.01f;
  a.c2 = 0.03f * 0.03f;
  float* part = (float*)d_workspace;
  float2* sums = (float2*)((char*)d_workspace + ssim_part_bytes(width, height));
  const dim3 grid((width + kSsimTile - 1) / kSsimTile, (height + kSsimTile - 1) / kSsimTile);
  hipStream_t s = (hipStream_t)stream;
  {
    TimedScope ts("loss_ssim", s);
    hipLaunchKernelGGL(k_ssim_stats, grid, dim3(kSsimTile * kSsimTile), 0, s, d_image, d_target, a, part, sums);
    hipLaunchKernelGGL(k_ssim_grad, grid, dim3(kSsimTile * kSsimTile), 0, s, d_image, d_target, a, part, sums,
                       (int32_t)(grid.x * grid.y), d_dL_dimage, d_loss);
  }
  return check_launch("gs_loss_l1_ssim");
}
