// L1 photometric loss and its gradient: the L1 term of section 7's training loss
// ((1 - lambda) L1 + lambda (1 - SSIM)) in "Gaussian splatting in PyTorch".
// L = mean |image - target| over h*w*3 values; dL/dimage = sign(image - target) / (3 h w).
// Elementwise and HBM-bound (8 B read + 4 B written per value); float4 vectorised when all three
// arrays are 16-byte aligned, scalar otherwise. The loss
// value, when asked for, is reduced per workgroup and added atomically into *loss (cleared first,
// in stream order), so its last bits may vary run to run.
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

}  // namespace
}  // namespace gs

using namespace gs;

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
