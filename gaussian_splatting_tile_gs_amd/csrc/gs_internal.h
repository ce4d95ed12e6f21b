// Internal declarations shared by the HIP translation units of libgs_hip.so (gfx950 only).
//
// The whole library is compiled with -ffp-contract=off: every fused multiply-add below is an
// explicit fmaf, so each expression rounds exactly as written. That makes the projection's
// integer results (radii, tile rectangles, tile counts) reproducible bit for bit, and makes the
// forward and backward raster kernels take identical skip/stop decisions, because they share
// the same inline evaluation of a splat at a pixel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "gs.h"

namespace gs {

// ---------------------------------------------------------------------------------------------
// Device-side camera: copied by value into kernel arguments.
// ---------------------------------------------------------------------------------------------
struct DevCamera {
  float V[16];
  float fx, fy, cx, cy;
  int32_t W, H;
  float near_plane;
  float bg[3];
  int32_t tiles_x, tiles_y;
  int32_t radius_mode, antialiased;  // the section-4 variants (0, 0: the default)
  int32_t tight_tiles;               // list only the tiles of the rectangle the ellipse reaches
};

inline DevCamera to_dev(const gs_camera& c) {
  DevCamera d;
  for (int i = 0; i < 16; ++i) d.V[i] = c.viewmat[i];
  d.fx = c.fx; d.fy = c.fy; d.cx = c.cx; d.cy = c.cy;
  d.W = c.width; d.H = c.height;
  d.near_plane = c.near_plane;
  d.bg[0] = c.background[0]; d.bg[1] = c.background[1]; d.bg[2] = c.background[2];
  d.tiles_x = (c.width + GS_TILE_SIZE - 1) / GS_TILE_SIZE;
  d.tiles_y = (c.height + GS_TILE_SIZE - 1) / GS_TILE_SIZE;
  d.radius_mode = c.radius_mode;
  d.antialiased = c.antialiased;
  d.tight_tiles = c.tight_tiles;
  return d;
}

// max/min with the exact semantics of (a < b) ? b : a and (b < a) ? b : a.
__host__ __device__ __forceinline__ float omax(float a, float b) { return (a < b) ? b : a; }
__host__ __device__ __forceinline__ float omin(float a, float b) { return (b < a) ? b : a; }

// Device-coherent accesses for data that other workgroups of the same launch read: relaxed
// atomic loads and stores at device scope go past the per-XCD L2 to the point where every XCD
// sees them, so no L2-wide write-back fence is needed. Once the issuing wave's memory counter has
// drained (wait_mem) such a store is visible to every workgroup, so a word read after a flag that
// was set behind it sees it.
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's memory operations have completed (a workgroup barrier does not: within
// a workgroup, memory is coherent without it). Before a device-scope flag store, it makes the
// device-coherent stores ahead of it visible to whoever sees the flag.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------------------------
// Reproducible fp32 exp and log for the activations.
// exp: Cody & Waite (1980) additive range reduction x = k ln2 + r, with ln2 split into a short
// head (exact products k * head) and a tail; e^r from the degree-7 Taylor polynomial by Horner's
// rule in fused multiply-adds; e^x = 2^k e^r. Input clamped to [-87, 88] (normal results).
// log: x = m 2^e, m moved into [sqrt(1/2), sqrt(2)); ln m = 2 atanh(s), s = (m - 1)/(m + 1),
// odd atanh series through s^9; ln x = e ln2 + ln m.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float act_exp(float x) {
  if (x != x) return x;
  x = (x < -87.0f) ? -87.0f : x;
  x = (x > 88.0f) ? 88.0f : x;
  const float k = rintf(x * 0x1.715476p+0f);
  const float r = (x - k * 0x1.62e4p-1f) - k * 0x1.7f7d1cp-20f;
  float p = 0x1.a01a02p-13f;
  p = fmaf(p, r, 0x1.6c16c2p-10f);
  p = fmaf(p, r, 0x1.111112p-7f);
  p = fmaf(p, r, 0x1.555556p-5f);
  p = fmaf(p, r, 0x1.555556p-3f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

__device__ __forceinline__ float act_log(float x) {
  if (x != x) return x;
  if (x < 0.0f) return __builtin_nanf("");
  if (x == 0.0f) return -__builtin_inff();
  if (x == __builtin_inff()) return x;
  int e = 0;
  float m = frexpf(x, &e);
  if (m < 0x1.6a09e6p-1f) {
    m = m * 2.0f;
    e = e - 1;
  }
  const float s = (m - 1.0f) / (m + 1.0f);
  const float s2 = s * s;
  float q = 0x1.c71c72p-4f;
  q = fmaf(q, s2, 0x1.24924ap-3f);
  q = fmaf(q, s2, 0x1.99999ap-3f);
  q = fmaf(q, s2, 0x1.555556p-2f);
  const float t = s2 * q;
  const float two_s = 2.0f * s;
  const float lnm = fmaf(two_s, t, two_s);
  const float fe = (float)e;
  const float r = fmaf(fe, 0x1.7f7d1cp-20f, lnm);
  return fmaf(fe, 0x1.62e4p-1f, r);
}

// Tile rectangle [x0, x1) x [y0, y1) of a splat with mean (mx, my) and radii (rx, ry), clamped
// to the grid; the same expression is used by the projection (to count) and by the emitter.
struct TileRect {
  int32_t x0, y0, x1, y1;
};
__device__ __forceinline__ TileRect tile_rect(float mx, float my, float rx, float ry, int32_t tiles_x,
                                              int32_t tiles_y) {
  float x0 = floorf((mx - rx) / 16.0f), x1 = ceilf((mx + rx) / 16.0f);
  float y0 = floorf((my - ry) / 16.0f), y1 = ceilf((my + ry) / 16.0f);
  x0 = omin(omax(x0, 0.0f), (float)tiles_x);
  x1 = omin(omax(x1, 0.0f), (float)tiles_x);
  y0 = omin(omax(y0, 0.0f), (float)tiles_y);
  y1 = omin(omax(y1, 0.0f), (float)tiles_y);
  return {(int32_t)x0, (int32_t)y0, (int32_t)x1, (int32_t)y1};
}

// ---------------------------------------------------------------------------------------------
// Tight tile rows (camera option tight_tiles): row ty of a splat's rectangle keeps the tiles
// [xs, xe) whose pixel-centre box [16 tx + 0.5, 16 tx + 15.5] x [16 ty + 0.5, 16 ty + 15.5]
// meets the ellipse sigma <= s2. No pixel centre beyond sigma = k^2 / 2 sees alpha >= 1/255
// (k = min(3.33, sqrt(2 ln(255 o))), section 4's extent), and s2 widens that level by
// 0.002 + s (0.002 + q / 65536), q = A C / (A C - B^2) >= 1 bounding the size of sigma's terms
// on the ellipse (4 s q), so that fp32 rounding in the blend's sigma or in these bounds cannot
// drop a reached pixel. With v = y - my over the row's centre rows (clipped to |v| <=
// sqrt(2 s2 A / D), D = A C - B^2) the ellipse spans u = x - mx in [L, R]: R is largest at
// v = -B t and L smallest at v = B t, t = sqrt(2 s2 / (C D)) (clamped into the row), with
// u = (-B v +- sqrt(2 s2 A - D v^2)) / A. Degenerate or extreme shapes (D <= 0, q >= 1e6,
// 2 s2 / D >= 1e30) keep the whole row. The projection counts with these functions, the binning
// lists with them and the deterministic backward indexes pairs with them: the same fp32 ops,
// contraction off, give the same tiles everywhere.
// ---------------------------------------------------------------------------------------------
struct TightShape {
  float mx, my, A, B, C, D, s2, E;
  bool full;  // keep every tile of the rectangle
};
__device__ __forceinline__ TightShape tight_shape(float mx, float my, float A, float B, float C, float o) {
  TightShape t;
  t.mx = mx;
  t.my = my;
  t.A = A;
  t.B = B;
  t.C = C;
  float kk = 2.0f * act_log(255.0f * o);
  if (!(kk > 0.0f)) kk = 0.0f;
  float k = sqrtf(kk);
  if (k > 3.33f) k = 3.33f;
  const float s = 0.5f * k * k;
  t.D = A * C - B * B;
  const float q = (A * C) / t.D;
  t.full = !(A > 0.0f) || !(C > 0.0f) || !(t.D > 0.0f) || !(q < 1e6f);
  t.s2 = 0.0f;
  t.E = 0.0f;
  if (!t.full) {
    t.s2 = s + (0.002f + s * (0.002f + q * 0x1p-16f));
    t.E = 2.0f * t.s2 / t.D;
    t.full = !(t.E < 1e30f);
  }
  return t;
}
// (xs, xe) of tile row ty inside the rectangle columns [x0, x1); xe == xs when the row is empty
__device__ __forceinline__ int2 tight_row(const TightShape& t, int ty, int x0, int x1) {
  if (t.full) return make_int2(x0, x1);
  const float ry = sqrtf(t.E * t.A), tt = sqrtf(t.E / t.C);
  const float ylo = ((float)(16 * ty) + 0.5f) - t.my, yhi = ((float)(16 * ty) + 15.5f) - t.my;
  const float lo = omax(ylo, -ry), hi = omin(yhi, ry);
  if (lo > hi) return make_int2(x0, x0);
  const float vr = omin(omax(-(t.B * tt), lo), hi);
  const float vl = omin(omax(t.B * tt, lo), hi);
  const float R = (-(t.B * vr) + sqrtf(omax(2.0f * t.s2 * t.A - t.D * vr * vr, 0.0f))) / t.A;
  const float L = (-(t.B * vl) - sqrtf(omax(2.0f * t.s2 * t.A - t.D * vl * vl, 0.0f))) / t.A;
  float xs = ceilf((t.mx + L - 15.5f) / 16.0f);
  float xe = floorf((t.mx + R - 0.5f) / 16.0f) + 1.0f;
  xs = omin(omax(xs, (float)x0), (float)x1);
  xe = omin(omax(xe, (float)x0), (float)x1);
  if (xe < xs) xe = xs;
  return make_int2((int)xs, (int)xe);
}

// ---------------------------------------------------------------------------------------------
// One splat evaluated at one pixel centre: the blend's sigma, alpha and its skip decision.
// The record stores the conic pre-scaled by log2(e) (hA = A/2 log2e, B2 = B log2e, hC = C/2
// log2e) so that exp(-sigma) is a single exp2. Forward and backward call this same function.
// ---------------------------------------------------------------------------------------------
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTransmittanceMin = 1e-4f;

struct SplatEval {
  float alpha;  // min(0.99, o G), meaningful when !skip
  float G;      // exp(-sigma)
  float s2;     // log2(e) sigma
  bool skip;    // sigma < 0 or alpha < 1/255
  bool capped;  // o G >= 0.99 (alpha is the constant cap: no gradient to o or sigma)
};

__device__ __forceinline__ SplatEval eval_splat(float dx, float dy, float hA, float B2, float hC, float o) {
  // s2 = log2(e) * sigma = dx (hA dx + B2 dy) + hC dy^2: five VALU operations
  const float s2 = fmaf(fmaf(hA, dx, B2 * dy), dx, (hC * dy) * dy);
  SplatEval e;
  e.s2 = s2;
  e.G = __builtin_amdgcn_exp2f(-s2);  // v_exp_f32; results below 2^-126 flush to 0 (alpha < 1/255)
  const float raw = o * e.G;          // never NaN: o in [0, 1], G in [0, inf)
  e.capped = raw >= kAlphaMax;
  e.alpha = fminf(raw, kAlphaMax);
  e.skip = (s2 < 0.0f) || (e.alpha < kAlphaMin);
  return e;
}

// ---------------------------------------------------------------------------------------------
// Raster plan (written by gs_bin_and_sort, read by the raster calls), u32 words:
//   [0] chunk length L, [1] X = extra work items, [2] checkpoint slots, [3] XF = split chunks,
//   [4, 4 + T)          tile processing order (T = number of tiles): slot 8 p + x holds place p of
//                       XCD x's list of tiles (plan_xcd), heaviest count class first, up to the
//                       shortest list's length m; the slots from 8 m on hold the longer lists' rest,
//   [4 + T, 4 + 2T)     per tile with two or more chunks, the index of its first checkpoint slot,
//   [4 + 2T, 4 + 2T + 2X)  the extra work items (tile, chunk >= 1),
//   [4 + 2T + 2M, 4 + 2T + 2M + 2XF)  (M = kPlanMaxChunks) the training forward's extra work
//                       items (tile, blended chunk >= 1) of the tiles it splits.
// A tile with c pairs has k = ceil(c / L) chunks of L list entries; when k >= 2 it has k slots,
// slot j holding, per pixel, the transmittance after chunk j and the colour that chunk j added.
// The backward's work items are the X extra ones, then, from the next multiple of 8 on (so that
// slot i runs on XCD i mod 8), (order[i], chunk 0) for every tile.
// L >= P / kPlanMaxChunks keeps X below kPlanMaxChunks and the slots below 2 kPlanMaxChunks.
// The training forward blends a tile of more than 512 entries and at least three chunks of 2 L
// entries chunk by chunk in parallel (plan_split): its work items are the XF split chunks, then
// (order[i], first chunk) for every tile, again from the next multiple of 8 on; XF < X / 2.
// ---------------------------------------------------------------------------------------------
constexpr uint32_t kPlanChunk = 0, kPlanExtra = 1, kPlanCheckpoints = 2, kPlanSplit = 3, kPlanOrder = 4;
// Workgroup b of a launch runs on XCD b mod 8, and each XCD has its own L2. A 128-B line of a 4-B
// per-pixel array holds 32 pixels of a row: the two tiles of a 2x1 block of tiles, which the order
// puts on one XCD. The blocks go round the XCDs along a row of blocks, each row of tiles shifted
// by three, so that every XCD gets a share of every part of the frame.
constexpr uint32_t kXcds = 8;
__host__ __device__ constexpr uint32_t plan_xcd(uint32_t t, uint32_t tiles_x) {
  return ((t % tiles_x) / 2u + 3u * (t / tiles_x)) % kXcds;
}
// The first work item of the tiles after n items before them: the next multiple of kXcds.
__host__ __device__ constexpr uint32_t plan_xcd_align(uint32_t n) { return (n + kXcds - 1u) / kXcds * kXcds; }
constexpr uint32_t kPlanMinChunk = 128;  // half a raster batch: boundaries fall where a mask word starts
constexpr uint32_t kPlanMaxChunks = 4096;
constexpr uint32_t kPlanMaxSlots = 2 * kPlanMaxChunks;
constexpr uint32_t kPlanMaxSplit = kPlanMaxChunks / 2;
// X < kPlanMaxChunks and XF < kPlanMaxSplit, so the aligned start of the tiles stays within the
// launches' extra workgroups (kPlanMaxChunks, kPlanMaxSplit)
static_assert(kPlanMaxChunks % kXcds == 0 && kPlanMaxSplit % kXcds == 0, "extra workgroups must align to the XCDs");
inline size_t plan_words(size_t ntiles) { return kPlanOrder + 2 * ntiles + 2 * kPlanMaxChunks + 2 * kPlanMaxSplit; }
// The training forward's split rule: the split's chain (a factor pass and a blend of one blended
// chunk of 2 L entries) must be well below the whole tile's walk to pay for the factor passes.
constexpr uint32_t kSplitMinChunks = 3, kSplitMinEntries = 513;
__host__ __device__ constexpr uint32_t plan_blended_chunks(uint32_t c, uint32_t L) { return (c + 2u * L - 1u) / (2u * L); }
__host__ __device__ constexpr bool plan_split(uint32_t c, uint32_t L) {
  return c >= kSplitMinEntries && plan_blended_chunks(c, L) >= kSplitMinChunks;
}
// The same for L = 2^lb (the binning's finalizer, where L is a power of two): shifts for divisions.
__host__ __device__ constexpr uint32_t plan_blended_chunks_pow2(uint32_t c, uint32_t lb) {
  return (c + (2u << lb) - 1u) >> (lb + 1u);
}
__host__ __device__ constexpr bool plan_split_pow2(uint32_t c, uint32_t lb) {
  return c >= kSplitMinEntries && plan_blended_chunks_pow2(c, lb) >= kSplitMinChunks;
}
static_assert(plan_split_pow2(512, 7) == plan_split(512, 128) && plan_split_pow2(513, 7) == plan_split(513, 128) &&
                  plan_split_pow2(768, 8) == plan_split(768, 256) && plan_split_pow2(1025, 8) == plan_split(1025, 256) &&
                  plan_blended_chunks_pow2(100000, 9) == plan_blended_chunks(100000, 512),
              "the power-of-two forms must agree with the general ones");

// ---------------------------------------------------------------------------------------------
// Host side: status, last error, kernel timing.
// ---------------------------------------------------------------------------------------------
gs_status set_error(gs_status s, const std::string& msg);
gs_status check_launch(const char* what);
bool valid_camera(const gs_camera* cam, std::string* why);

// Kernel timing: bracket a launch with events when enabled.
void timing_begin(const char* name, hipStream_t stream);
void timing_end(hipStream_t stream);

struct TimedScope {
  hipStream_t s;
  TimedScope(const char* name, hipStream_t stream) : s(stream) { timing_begin(name, stream); }
  ~TimedScope() { timing_end(s); }
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace gs
