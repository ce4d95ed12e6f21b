// Forward blend (k-blend), backward raster (k-rbwd) and backward projection (k-pbwd).
//
// Forward ("Gaussian splatting in PyTorch", section 5): per pixel, front to back over its tile's
// sorted list, alpha = min(0.99, o exp(-sigma)), skip below 1/255 or for sigma < 0, stop before
// adding once T (1 - alpha) <= 1e-4, finally add T * background.
// Backward (section 6; the production kernels "write the backward pass by hand, back to front"
// and recover T_i by dividing by 1 - alpha_j): per pixel back to front from its last
// contributor, with the weights recomputed rather than stored.
//
// MI355X design:
//  - one 256-thread workgroup (4 wave64) per 16 x 16 tile, one pixel per thread, wave q owning
//    the 8 x 8 quadrant q; Gaussians are staged 256 at a time in LDS as pre-scaled records (every
//    lane then reads the same record: an LDS broadcast, no bank conflicts);
//  - the loaders mark which quadrants each staged splat's ellipse reaches at alpha >= 1/255
//    (64-lane ballots into four 256-bit masks); a wave walks only its mask's set bits, with a wave-uniform scalar loop,
//    and a predicated (branch-free) body;
//  - a wave leaves the batch as soon as all 64 of its pixels are done (wave-uniform test), the
//    workgroup stops loading batches when all 256 are (__syncthreads_count);
//  - workgroup b takes tile order[b] when a processing order is given (heaviest tiles first, so
//    the longest workgroups start first and do not end the kernel alone), else tile b;
//  - backward: nine per-lane terms per splat (linear pieces of its 2D gradient) are summed over
//    the wave by a reduce-scatter of permlane swaps and DPP exchanges (25 VALU ops in all),
//    accumulated per workgroup in LDS (ds_add_f32), turned into the 2D gradient and flushed once
//    per (tile, splat) with global fp32 atomics.
// Both raster kernels evaluate a splat with the same inline eval_splat, so the backward takes
// exactly the forward's skip decisions.
#include <type_traits>

#include "project_core.h"

namespace gs {
namespace {

constexpr int kTile = 16;
constexpr int kRasterThreads = kTile * kTile;  // 256: one pixel per thread
constexpr int kBatch = kRasterThreads;         // splats staged per batch
// chunk lengths are powers of two >= kPlanMinChunk: a boundary falls on a batch start or on the
// start of a 64-splat word of the quadrant masks, where each wave can store its pixels' state
static_assert(kBatch % kPlanMinChunk == 0 && kPlanMinChunk % 64 == 0, "chunk boundaries must fall on mask words");

// Staged splat record: (mx, my, hA, hC), (B2, o, r, g), (b, z, 0, 0). hA = A/2 log2e, B2 = B log2e,
// hC = C/2 log2e, so that log2(e) sigma = hA dx^2 + hC dy^2 + B2 dx dy. Staging also returns the
// 4-bit set of 8x8 quadrants of the tile where the splat can reach alpha >= 1/255 at some pixel
// centre (its ellipse at that level meets the quadrant); elsewhere it skips at every pixel.
// The test uses the splat alone, not its radii, so it holds for every radius rule.
// An id >= n (impossible for a well-formed sorted list) stages a record that never contributes.
//
// The raw record of one splat is loaded into registers first (in the blend a batch ahead of its
// staging, so that its loads are in flight while the previous batch is walked). The three parts
// sit in three arrays of 16-B entries, so that a walk reads all of splat k's record from one
// address register (k times 16) with three offsets; the backward with a depth channel keeps the
// third part in 8-B entries, (b, z), for its LDS budget. z is 0 without a depth channel.
struct RawSplat {
  float2 m;
  float A, B, C, o, r, g, b, z;
};
template <bool DEPTH>
__device__ __forceinline__ RawSplat load_raw(uint32_t g, uint32_t n, const float* __restrict__ means2d,
                                             const float* __restrict__ conics, const float* __restrict__ opac,
                                             const float* __restrict__ colors, const float* __restrict__ depths) {
  RawSplat s;
  if (g >= n) {  // past the list, or an id that cannot be: zero opacity, never contributes
    s.m = make_float2(0.0f, 0.0f);
    s.B = s.o = s.r = s.g = s.b = s.z = 0.0f;
    s.A = s.C = 1.0f;
    return s;
  }
  s.m = *reinterpret_cast<const float2*>(means2d + 2 * g);
  s.A = conics[3 * g];
  s.B = conics[3 * g + 1];
  s.C = conics[3 * g + 2];
  s.o = opac[g];
  s.r = colors[3 * g];
  s.g = colors[3 * g + 1];
  s.b = colors[3 * g + 2];
  s.z = DEPTH ? depths[g] : 0.0f;
  return s;
}

// Stages a raw record: the pre-scaled LDS record (a, b, c) and the quadrant mask (0 when not
// valid). Exact test of the splat's ellipse against each quadrant: the minimum over the
// quadrant's box of pixel centres of s2 = log2(e) sigma (a positive definite quadratic in the
// offset, so the minimum is 0 inside the box and otherwise lies on an edge, where it is a 1D
// quadratic) must not exceed log2(255 o), else alpha < 1/255 at every pixel centre of the
// quadrant. The slack (0.02 + 4e-6 times the size of the quadratic's terms over the tile) is far
// above the fp32 rounding of both this bound and the evaluation's s2, so no contributing splat is
// dropped.
__device__ __forceinline__ void put_bz(float4& c, float b, float z) { c = make_float4(b, z, 0.0f, 0.0f); }
__device__ __forceinline__ void put_bz(float2& c, float b, float z) { c = make_float2(b, z); }
template <typename BZ>
__device__ __forceinline__ uint32_t stage_raw(const RawSplat& rs, bool valid, float tx0, float ty0, float4& a,
                                              float4& b, BZ& c) {
  a = make_float4(rs.m.x, rs.m.y, (0.5f * kLog2e) * rs.A, (0.5f * kLog2e) * rs.C);
  b = make_float4(kLog2e * rs.B, rs.o, rs.r, rs.g);
  put_bz(c, rs.b, rs.z);
  if (!valid) return 0u;
  const float qa = a.z, qb = b.x, qc = a.w;  // hA, B2, hC
  const float ia = 0.5f / qa, ic = 0.5f / qc;
  const float ex0 = tx0 + 0.5f - rs.m.x, ey0 = ty0 + 0.5f - rs.m.y;  // offsets of the tile's first centre
  const float X = fmaxf(fabsf(ex0), fabsf(ex0 + 15.0f)), Y = fmaxf(fabsf(ey0), fabsf(ey0 + 15.0f));
  const float terms = fmaf(qa * X, X, fmaf(fabsf(qb) * X, Y, (qc * Y) * Y));
  const float lim = __log2f(255.0f * b.y) + fmaf(4e-6f, terms, 0.02f);
  auto q2 = [&](float x, float y) { return fmaf(fmaf(qa, x, qb * y), x, (qc * y) * y); };
  uint32_t qm = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x_lo = tx0 + (float)((q & 1) * 8) + 0.5f, y_lo = ty0 + (float)((q >> 1) * 8) + 0.5f;
    const float x0 = x_lo - rs.m.x, x1 = x0 + 7.0f, y0 = y_lo - rs.m.y, y1 = y0 + 7.0f;
    // on the edge x = e the minimiser is y = -B2 e / (2 hC), clamped; likewise on y = e
    const float s_l = q2(x0, fminf(fmaxf(-qb * x0 * ic, y0), y1));
    const float s_r = q2(x1, fminf(fmaxf(-qb * x1 * ic, y0), y1));
    const float s_t = q2(fminf(fmaxf(-qb * y0 * ia, x0), x1), y0);
    const float s_b = q2(fminf(fmaxf(-qb * y1 * ia, x0), x1), y1);
    const bool in = x0 <= 0.0f && x1 >= 0.0f && y0 <= 0.0f && y1 >= 0.0f;
    const bool hit = in || fminf(fminf(s_l, s_r), fminf(s_t, s_b)) <= lim;
    qm |= hit ? (1u << q) : 0u;
  }
  return qm;
}

// Sum over the 64 lanes of a wave with DPP; the total lands in lane 63 (other lanes hold partial
// sums). Row shifts with bound_ctrl read 0 past a row's start, so no row/bank masking is needed
// for lane 63's result, and every step folds into one v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
  float r = v + dpp_f<0x111>(v);  // row_shr:1
  r = r + dpp_f<0x112>(v);        // row_shr:2
  r = r + dpp_f<0x113>(v);        // row_shr:3 -> lane i: v[i-3..i] within its row
  r = r + dpp_f<0x114>(r);        // row_shr:4 -> v[i-7..i]
  r = r + dpp_f<0x118>(r);        // row_shr:8 -> lane 15 of each row holds the row's sum
  r = r + dpp_f<0x142>(r);        // row_bcast:15 -> lane 63 holds rows 2 + 3, lane 31 rows 0 + 1
  r = r + dpp_f<0x143>(r);        // row_bcast:31 -> lane 63 holds the wave
  return r;
}

// Maximum over the 64 lanes of a wave, into lane 63 (same DPP pattern; 0 is the identity).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_max_lane63(uint32_t v) {
  uint32_t r = max(v, dpp_u<0x111>(v));
  r = max(r, dpp_u<0x112>(v));
  r = max(r, dpp_u<0x113>(v));
  r = max(r, dpp_u<0x114>(r));
  r = max(r, dpp_u<0x118>(r));
  r = max(r, dpp_u<0x142>(r));
  r = max(r, dpp_u<0x143>(r));
  return r;
}

// Adds the workgroup's evaluation count to *eval_count: one atomic per workgroup.
__device__ __forceinline__ void count_evals(uint32_t n_eval, unsigned long long* eval_count) {
  __shared__ uint32_t s_cnt;
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
  const float tot = wave_sum_lane63((float)n_eval);
  if ((threadIdx.x & 63) == 63 && tot > 0.0f) atomicAdd(&s_cnt, (uint32_t)(tot + 0.5f));
  __syncthreads();
  if (threadIdx.x == 0 && s_cnt) atomicAdd(eval_count, (unsigned long long)s_cnt);
}

// A wave-uniform 64-bit value read from LDS, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Per batch, the loaders publish one 64-bit ballot per (quadrant, loading wave): bit j of
// s_qm[q][w] says that staged splat 64 w + j reaches quadrant q. Wave q then walks its set bits.
__device__ __forceinline__ void publish_quadrant_masks(uint32_t qm, bool valid, uint64_t (*s_qm)[4]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t b = __ballot(valid && ((qm >> q) & 1u));
    if (lane == 0) s_qm[q][wave] = b;
  }
}

// Per-lane flags as wave-uniform lane masks (bit l: lane l), kept in scalar registers, so that
// testing, combining and setting them costs no vector instruction: lane_in(m) is this lane's bit,
// lanes_where(c) the mask of the lanes where c holds (of a single compare, it is that compare's
// own result).
__device__ __forceinline__ bool lane_in(uint64_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }
__device__ __forceinline__ uint64_t lanes_where(bool c) { return __builtin_amdgcn_ballot_w64(c); }
// The lanes where a splat is skipped (sigma < 0 or alpha < 1/255), one mask per compare.
__device__ __forceinline__ uint64_t lanes_skipped(const SplatEval& e) {
  return lanes_where(e.s2 < 0.0f) | lanes_where(e.alpha < kAlphaMin);
}

// One front-to-back blend step of a pixel (section 5's loop body, predicated). DEPTH: the depth
// channel (the splat's camera z) goes through the same weight.
template <bool DEPTH>
__device__ __forceinline__ void blend_step(const SplatEval& e, bool act, float cr_, float cg_, float cb_, float z_,
                                           uint32_t idx, float& T, float& cr, float& cg, float& cb, float& cd,
                                           uint32_t& last, bool& done) {
  const bool ok = act && !done && !e.skip;
  const float nT = T * (1.0f - e.alpha);
  // nT >= 0, so comparing its bits as integers orders it like the float, and, unlike a float
  // compare (NaN), the negation is free: one compare serves both outcomes
  const bool low = __float_as_uint(nT) <= __float_as_uint(kTransmittanceMin);
  const bool stop = ok && low;
  const bool add = ok && !low;
  const float Tn = add ? nT : T;
  const float wgt = T - Tn;  // alpha T when added (to rounding), exactly 0 otherwise
  cr = fmaf(cr_, wgt, cr);
  cg = fmaf(cg_, wgt, cg);
  cb = fmaf(cb_, wgt, cb);
  if (DEPTH) cd = fmaf(z_, wgt, cd);
  T = Tn;
  last = add ? idx : last;
  done = done || stop;
}

// ---------------------------------------------------------------------------------------------
// k-blend: one 256-thread workgroup per 16x16 tile; wave q owns the 8x8 quadrant q and walks its
// splats two per iteration (their alphas are independent; the T updates are sequential). With a
// raster plan, workgroup b takes tile order[b].
// CHUNKED (a plan and the raster workspace: a training forward): the backward splits a tile longer
// than the plan's chunk length L into chunks of L list entries, so the forward stores for every
// chunk j, per pixel, the transmittance after the chunk and the colour (and depth) it added
// (checkpoint slot j of the tile); each wave stores its own pixels' slot as it passes a boundary,
// where the boundary's 64-splat mask word starts. A tile that is not split is walked by one
// workgroup. A tile of three or more blended chunks of 2 L entries and more than 512 entries is
// split: its blended chunks run at once, one workgroup each (the plan's extra work items
// (tile, j) of even j >= 2, and the tile's own workgroup for the first). The workgroup of blended
// chunk c >= 1 first forms the transmittance factor of blended chunk c - 1 (the product of
// 1 - alpha over its contributing splats, no stop rule; a factor that falls to 1e-4 or below stays
// there) and publishes it, then waits for the factors of blended chunks 0 .. c - 2 published by
// the workgroups of blended chunks 1 .. c - 1, starts from their product and blends its chunk,
// storing the slots of its two plan chunks. A pixel that stopped in an earlier chunk starts at or
// below 1e-4 and so adds nothing. The last of a split tile's workgroups to finish forms its
// pixels: the transmittance of the first plan chunk that stopped (else of the last chunk), the
// colours summed over the chunks in order, the last added entry of the last chunk that added one.
// The chunk workgroups take tickets in launch order, so a workgroup only waits for workgroups that
// have started; every wait is also bounded.
// DEPTH: also the depth channel, D = sum z_i alpha_i T_i (background depth 0).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float l1_sign(float d) { return d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f); }

constexpr uint32_t kWaitPolls = 1u << 22;    // a bound on each wait for a published factor

// The raster workspace, per checkpoint slot and pixel: (T after the chunk, colour the chunk added),
// the depth the chunk added, the transmittance factor of the chunk, the chunk's last added entry
// with bit 31 set when the pixel stopped in it. Then the chunked forward's synchronisation words:
// [0] ticket counter, [1] finished ticketed workgroups, per slot an arrival counter (used at a
// split tile's first slot) and a published-factor flag. They are zero between calls (the last
// ticketed workgroup resets the two counters, a split tile's last workgroup its own words), so
// the workspace is zeroed once before its first use.
struct RasterWs {
  float4* ckpt;
  float* ckpt_d;
  float* tprod;
  uint32_t* lastc;
  uint32_t* sync;
};
constexpr size_t kRasterSyncWords = 2 + 2 * (size_t)kPlanMaxSlots;
__host__ __device__ inline RasterWs raster_ws_parts(void* base) {
  RasterWs w{};
  if (!base) return w;
  const size_t px = (size_t)kPlanMaxSlots * 256;
  w.ckpt = (float4*)base;
  w.ckpt_d = (float*)(w.ckpt + px);
  w.tprod = w.ckpt_d + px;
  w.lastc = (uint32_t*)(w.tprod + px);
  w.sync = w.lastc + px;
  return w;
}

// Walks list entries [rs, re) of a tile (staged 256 at a time, the next batch's records loading
// while a batch is walked) and calls visit(k0, k1, has1, list1) for the staged splats reaching the
// wave's quadrant, two per call; stops when every pixel of the workgroup is done. at_word(e) is
// called by each wave before it walks a 64-splat word of its mask (wave-uniform), with the word's
// first list entry.
template <bool DEPTH, typename VISIT, typename AT_WORD>
__device__ __forceinline__ void walk_entries(uint32_t n, const uint32_t* __restrict__ ids, uint32_t start, uint32_t rs,
                                             uint32_t re, const float* __restrict__ means2d,
                                             const float* __restrict__ conics, const float* __restrict__ opac,
                                             const float* __restrict__ colors, const float* __restrict__ depths,
                                             float tx0, float ty0, const bool& done, float4* s_a, float4* s_b,
                                             float4* s_c, uint64_t (*s_qm)[4], VISIT visit,
                                             AT_WORD at_word) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint32_t b0 = start + rs, e0 = start + re;
  uint32_t id_next2 = b0 + kBatch + tid < e0 ? ids[b0 + kBatch + tid] : n;
  RawSplat raw = load_raw<DEPTH>(b0 + tid < e0 ? ids[b0 + tid] : n, n, means2d, conics, opac, colors, depths);
  for (uint32_t bs = b0; bs < e0; bs += kBatch) {
    if (__syncthreads_count(done) == kRasterThreads) break;
    const bool valid = bs + tid < e0;
    const uint32_t qm = stage_raw(raw, valid, tx0, ty0, s_a[tid], s_b[tid], s_c[tid]);
    publish_quadrant_masks(qm, valid, s_qm);
    {
      const uint32_t j2 = bs + 2 * kBatch + tid;
      raw = load_raw<DEPTH>(id_next2, n, means2d, conics, opac, colors, depths);
      id_next2 = j2 < e0 ? ids[j2] : n;
    }
    __syncthreads();
    const uint32_t list1 = bs - start + 1u;  // 1-based list index of staged splat 0
    for (int w = 0; w < 4; ++w) {
      at_word(bs - start + (uint32_t)(w * 64));
      uint64_t m = uniform64(s_qm[wave][w]);
      while (m) {
        if (!__any(!done)) break;
        const int bit0 = __builtin_ctzll(m);
        m &= m - 1;
        const bool has1 = m != 0;
        const int bit1 = has1 ? __builtin_ctzll(m) : bit0;
        if (has1) m &= m - 1;
        visit(w * 64 + bit0, w * 64 + bit1, has1, list1);
      }
    }
  }
}

template <bool COUNT, bool CHUNKED, bool DEPTH>
__global__ __launch_bounds__(kRasterThreads) void k_blend(
    uint32_t n, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ plan, uint32_t ntiles, RasterWs ws,
    const uint32_t* __restrict__ ids, const float* __restrict__ means2d, const float* __restrict__ conics,
    const float* __restrict__ opac, const float* __restrict__ colors, const float* __restrict__ depths,
    DevCamera cam, float* __restrict__ image, float* __restrict__ depth_out, float* __restrict__ final_T,
    uint32_t* __restrict__ n_contrib, unsigned long long* __restrict__ eval_count,
    const float* __restrict__ l1_target, float* __restrict__ l1_grad, float l1_scale) {
  __shared__ float4 s_a[kBatch];
  __shared__ float4 s_b[kBatch];
  __shared__ float4 s_c[kBatch];
  __shared__ uint64_t s_qm[4][4];
  __shared__ uint32_t s_word;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tile = -1;
  uint32_t chunk = 0, nx = 0;
  bool ticketed = false;
  if (CHUNKED) {
    nx = plan[kPlanSplit];
    if (blockIdx.x < nx) {
      // a split chunk: its ticket picks the item, so items are taken in the order they start
      if (tid == 0) s_word = atomicAdd(&ws.sync[0], 1u);
      __syncthreads();
      const uint32_t b = s_word;
      ticketed = true;
      if (b < nx) {  // always, with the counters zero at the launch
        const uint32_t* item = plan + kPlanOrder + 2 * ntiles + 2 * kPlanMaxChunks + 2 * b;
        tile = (int)item[0];
        chunk = 2u * item[1];  // the plan chunk that starts the blended chunk
      }
    } else {
      // the tiles from a multiple of 8 on: order slot i runs on XCD i mod 8
      const uint32_t b0 = plan_xcd_align(nx);
      if (blockIdx.x < b0 || blockIdx.x - b0 >= ntiles) return;  // workgroup-uniform
      tile = (int)plan[kPlanOrder + blockIdx.x - b0];
    }
  } else {
    tile = plan ? (int)plan[kPlanOrder + blockIdx.x] : (int)blockIdx.x;
  }
  uint32_t n_eval = 0;
  if (tile >= 0) {
    const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
    const float tx0 = (float)(tx * kTile), ty0 = (float)(ty * kTile);
    const int px_i = tx * kTile + (wave & 1) * 8 + (lane & 7);
    const int py_i = ty * kTile + (wave >> 1) * 8 + (lane >> 3);
    const bool inside = px_i < cam.W && py_i < cam.H;
    const float px = (float)px_i + 0.5f, py = (float)py_i + 0.5f;
    // the fused L1's target, loaded now so that the finished pixel does not wait for it
    float tr = 0.0f, tg = 0.0f, tb = 0.0f;
    if (l1_target && inside) {
      const int p = py_i * cam.W + px_i;
      tr = l1_target[3 * p + 0];
      tg = l1_target[3 * p + 1];
      tb = l1_target[3 * p + 2];
    }
    const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
    const uint32_t len = end - start;
    const uint32_t L = CHUNKED ? plan[kPlanChunk] : 1u;
    const uint32_t nch = (CHUNKED && len > L) ? (len + L - 1u) / L : 1u;  // the plan's chunks
    // a split tile is blended in chunks of two plan chunks (the split pays only for long chains;
    // the backward's chunks stay short), fc of them
    const uint32_t Lf = 2u * L;
    const uint32_t nf = plan_blended_chunks(len, L);
    const bool split = CHUNKED && plan_split(len, L);
    const uint32_t fc = chunk >> 1;  // the blended chunk that plan chunk `chunk` belongs to
    const uint32_t sbase = nch > 1 ? plan[kPlanOrder + ntiles + tile] : 0u;  // the tile's first slot
    // the items are the split tiles' blended chunks; a tile's own workgroup takes its first one
    // (all of it when it is not split)
    {
      const uint32_t rs = split ? fc * Lf : 0u;
      const uint32_t re = split ? (rs + Lf < len ? rs + Lf : len) : len;
      float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f, cd = 0.0f;
      if (split && fc > 0) {
        // the factor of blended chunk fc - 1, published for the later ones
        float F = 1.0f;
        bool fdone = !inside;
        walk_entries<false>(n, ids, start, rs - Lf, rs, means2d, conics, opac, colors, depths, tx0, ty0, fdone, s_a,
                            s_b, s_c, s_qm, [&](int k0, int k1, bool has1, uint32_t) {
          const float4 a0 = s_a[k0], b0 = s_b[k0];
          const float4 a1 = s_a[k1], b1 = s_b[k1];
          const SplatEval e0 = eval_splat(a0.x - px, a0.y - py, a0.z, b0.x, a0.w, b0.y);
          const SplatEval e1 = eval_splat(a1.x - px, a1.y - py, a1.z, b1.x, a1.w, b1.y);
          F = (!fdone && !e0.skip) ? F * (1.0f - e0.alpha) : F;
          F = (has1 && !fdone && !e1.skip) ? F * (1.0f - e1.alpha) : F;
          fdone = fdone || __float_as_uint(F) <= __float_as_uint(kTransmittanceMin);
        }, [](uint32_t) {});
        // published with device-coherent stores, complete before the barrier and so before the flag
        if (inside) st_dev(ws.tprod + (size_t)(sbase + fc - 1u) * kRasterThreads + tid, F);
        wait_mem();
        __syncthreads();
        if (tid == 0) {
          uint32_t* flag = ws.sync + 2 + kPlanMaxSlots + sbase;
          st_dev(flag + fc - 1u, 1u);
          for (uint32_t i = 0; i + 1u < fc; ++i) {
            uint32_t polls = 0;
            while (ld_dev(flag + i) == 0u && ++polls < kWaitPolls) __builtin_amdgcn_s_sleep(2);
          }
        }
        __syncthreads();
        if (inside) {
          for (uint32_t i = 0; i + 1u < fc; ++i) T *= ld_dev(ws.tprod + (size_t)(sbase + i) * kRasterThreads + tid);
          T *= F;
        }
      }
      uint32_t last = 0;
      // a chunk that starts at or below 1e-4 would stop at its first contributing splat: done already
      bool done = !inside || __float_as_uint(T) <= __float_as_uint(kTransmittanceMin);
      // the walk stores the slot of plan chunk j as it passes the start of chunk j + 1 (each wave
      // its own pixels, where the boundary's mask word starts); a blended chunk of a split tile
      // stores its plan chunks' slots device-coherently (another workgroup sums them), with the
      // last added entry and the stop bit; (pr, pg, pb, pd) hold the colour of the chunks before
      // the current one
      float pr = 0.0f, pg = 0.0f, pb = 0.0f, pd = 0.0f;
      const bool ckpts = CHUNKED && nch > 1;
      uint32_t next_b = (ckpts && rs + L < re) ? rs + L : 0xFFFFFFFFu;
      const size_t slot0 = (size_t)sbase * kRasterThreads + tid;
      size_t cur = slot0 + (split ? (size_t)(2u * fc) * kRasterThreads : 0u);  // the slot being filled
      auto put_slot = [&]() {
        if (!inside) return;
        if (split) {
          float* ck = (float*)(ws.ckpt + cur);
          st_dev(ck + 0, T);
          st_dev(ck + 1, cr);
          st_dev(ck + 2, cg);
          st_dev(ck + 3, cb);
          if (DEPTH) st_dev(ws.ckpt_d + cur, cd);
          st_dev(ws.lastc + cur, last | (done ? 0x80000000u : 0u));
        } else {
          ws.ckpt[cur] = make_float4(T, cr, cg, cb);
          if (DEPTH) ws.ckpt_d[cur] = cd;
        }
      };
      auto store_ckpt = [&]() {
        put_slot();
        cur += kRasterThreads;
        pr += cr;
        pg += cg;
        pb += cb;
        pd += cd;
        cr = cg = cb = cd = 0.0f;
        next_b += L;
        if (next_b >= re) next_b = 0xFFFFFFFFu;
      };
      walk_entries<DEPTH>(n, ids, start, rs, re, means2d, conics, opac, colors, depths, tx0, ty0, done, s_a, s_b,
                          s_c, s_qm, [&](int k0, int k1, bool has1, uint32_t list1) {
        const float4 a0 = s_a[k0], b0 = s_b[k0];
        const float4 a1 = s_a[k1], b1 = s_b[k1];
        const float2 cz0 = *reinterpret_cast<const float2*>(&s_c[k0]);
        const float2 cz1 = *reinterpret_cast<const float2*>(&s_c[k1]);
        const float c0 = cz0.x, c1 = cz1.x;
        const float z0 = DEPTH ? cz0.y : 0.0f, z1 = DEPTH ? cz1.y : 0.0f;
        const SplatEval e0 = eval_splat(a0.x - px, a0.y - py, a0.z, b0.x, a0.w, b0.y);
        const SplatEval e1 = eval_splat(a1.x - px, a1.y - py, a1.z, b1.x, a1.w, b1.y);
        if (COUNT) n_eval += (done ? 0u : 1u) + ((done || !has1) ? 0u : 1u);
        blend_step<DEPTH>(e0, true, b0.z, b0.w, c0, z0, list1 + (uint32_t)k0, T, cr, cg, cb, cd, last, done);
        blend_step<DEPTH>(e1, has1, b1.z, b1.w, c1, z1, list1 + (uint32_t)k1, T, cr, cg, cb, cd, last, done);
      }, [&](uint32_t e) {
        if (ckpts && e >= next_b) store_ckpt();  // wave-uniform
      });
      if (ckpts) {
        while (next_b != 0xFFFFFFFFu) store_ckpt();  // boundaries past the last walked batch
        put_slot();                                  // the last plan chunk's slot
        cr += pr;
        cg += pg;
        cb += pb;
        cd += pd;
      }
      bool finish = !split;
      if (split) {
        // the slots are out (device-coherent, complete before the barrier and so before the
        // arrival); the tile's last blended chunk to get here forms its pixels
        wait_mem();
        __syncthreads();
        if (tid == 0) s_word = atomicAdd(ws.sync + 2 + sbase, 1u);
        __syncthreads();
        finish = s_word == nf - 1u;
        if (finish) {
          T = 1.0f;
          cr = cg = cb = cd = 0.0f;
          last = 0;
          bool stopped = false;
          for (uint32_t c = 0; c < nch && inside; ++c) {
            const size_t oc = slot0 + (size_t)c * kRasterThreads;
            const float* ck = (const float*)(ws.ckpt + oc);
            const float sT = ld_dev(ck + 0);
            cr += ld_dev(ck + 1);
            cg += ld_dev(ck + 2);
            cb += ld_dev(ck + 3);
            const uint32_t lc = ld_dev(ws.lastc + oc);
            if (DEPTH) cd += ld_dev(ws.ckpt_d + oc);
            last = max(last, lc & 0x7FFFFFFFu);
            if (!stopped) T = sT;  // the first chunk that stopped holds the final transmittance
            stopped = stopped || (lc >> 31) != 0u;
          }
          // every workgroup of the tile has arrived, so no one reads its words any more
          if (tid == 0) st_dev(ws.sync + 2 + sbase, 0u);
          for (uint32_t i = tid; i + 1u < nf; i += kRasterThreads) st_dev(ws.sync + 2 + kPlanMaxSlots + sbase + i, 0u);
        }
      }
      if (finish && inside) {
        const int p = py_i * cam.W + px_i;
        const float ir = fmaf(T, cam.bg[0], cr), ig = fmaf(T, cam.bg[1], cg), ib = fmaf(T, cam.bg[2], cb);
        image[3 * p + 0] = ir;
        image[3 * p + 1] = ig;
        image[3 * p + 2] = ib;
        if (l1_target) {  // uniform: the L1 gradient sign(image - target) / (3 h w), as gs_loss_l1 forms it
          l1_grad[3 * p + 0] = l1_sign(ir - tr) * l1_scale;
          l1_grad[3 * p + 1] = l1_sign(ig - tg) * l1_scale;
          l1_grad[3 * p + 2] = l1_sign(ib - tb) * l1_scale;
        }
        final_T[p] = T;
        n_contrib[p] = last;
        if (DEPTH) depth_out[p] = cd;  // background depth 0
      }
    }
  }
  if (COUNT) count_evals(n_eval, eval_count);
  if (CHUNKED && ticketed && tid == 0) {
    // the last ticketed workgroup to finish: every ticket has been taken, so the counters reset
    if (atomicAdd(ws.sync + 1, 1u) == nx - 1u) {
      st_dev(ws.sync + 0, 0u);
      st_dev(ws.sync + 1, 0u);
    }
  }
}

// gfx950 lane exchanges: v_permlane32_swap trades lanes 32-63 of its first operand for lanes 0-31
// of its second (a' = [a.lo, b.lo], b' = [a.hi, b.hi]); v_permlane16_swap trades the odd 16-lane
// rows of the first for the even rows of the second (a' = [a.r0, b.r0, a.r2, b.r2],
// b' = [a.r1, b.r1, a.r3, b.r3]).
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t x = r[0], y = r[1];
  return __uint_as_float(x) + __uint_as_float(y);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t x = r[0], y = r[1];
  return __uint_as_float(x) + __uint_as_float(y);
}
template <int CTRL>
__device__ __forceinline__ float dppx(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// Adds the nine per-lane terms v[0..8] of one splat, summed over the wave, into acc[0..8] (LDS).
// Terms 0-7 go through a reduce-scatter: a permlane32 swap + add leaves term j in the low half
// and term j + 4 in the high half of one register (summed over lanes l, l ^ 32); a permlane16
// swap + add leaves terms j, j + 2, j + 4, j + 6 in rows 0-3 (summed over the four rows); a
// row_ror:8 exchange splits each row between two terms; three DPP adds finish each 8-lane group,
// so lane 8t holds term t: 18 VALU ops for eight terms, and the eight LDS atomics hit distinct
// addresses. Term 8 is summed with row shifts and row broadcasts into lane 63.
template <bool STORE>
__device__ __forceinline__ void reduce9_to_lds(const float* v, float* acc, int lane) {
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = swap32_sum(v[j], v[j + 4]);
  const float w0 = swap16_sum(u[0], u[2]);  // rows: terms 0, 2, 4, 6
  const float w1 = swap16_sum(u[1], u[3]);  // rows: terms 1, 3, 5, 7
  const bool hi = (lane & 8) != 0;
  float x = (hi ? w1 : w0) + dppx<0x128>(hi ? w0 : w1);  // row_ror:8: lanes l <-> l ^ 8
  x = x + dppx<0x141>(x);                                // row_half_mirror: l <-> 7 - l
  x = x + dppx<0x4E>(x);                                 // quad_perm [2,3,0,1]: l <-> l ^ 2
  x = x + dppx<0xB1>(x);                                 // quad_perm [1,0,3,2]: l <-> l ^ 1
  const float y = wave_sum_lane63(v[8]);
  if (STORE) {  // the wave's own slot: plain stores
    if ((lane & 7) == 0) acc[lane >> 3] = x;
    if (lane == 63) acc[8] = y;
  } else {
    if ((lane & 7) == 0) unsafeAtomicAdd(acc + (lane >> 3), x);
    if (lane == 63) unsafeAtomicAdd(acc + 8, y);
  }
}

// Slot of the pair (Gaussian g, tile (tx, ty)) in the per-pair gradient records: the pairs of a
// Gaussian are contiguous from base[g] (the exclusive prefix sum of tiles_touched in id order),
// in row-major order over its tile rectangle (the rectangle of the projection and the emitter; with
// tight tiles only the tiles of each row's tight run).
__device__ __forceinline__ uint32_t pair_slot(uint32_t g, const float* __restrict__ means2d,
                                              const int32_t* __restrict__ radii, const uint32_t* __restrict__ base,
                                              int tx, int ty, const DevCamera& cam, float A, float B, float C,
                                              float o) {
  const float2 m = *reinterpret_cast<const float2*>(means2d + 2 * g);
  const int2 r = *reinterpret_cast<const int2*>(radii + 2 * g);
  const TileRect rc = tile_rect(m.x, m.y, (float)r.x, (float)r.y, cam.tiles_x, cam.tiles_y);
  if (!cam.tight_tiles) return base[g] + (uint32_t)((ty - rc.y0) * (rc.x1 - rc.x0) + (tx - rc.x0));
  // tight tiles: the runs of the rows above, then the place in this row's run
  const TightShape ts = tight_shape(m.x, m.y, A, B, C, o);
  uint32_t local = 0;
  for (int y = rc.y0; y < ty; ++y) {
    const int2 sp = tight_row(ts, y, rc.x0, rc.x1);
    local += (uint32_t)(sp.y - sp.x);
  }
  const int2 sp = tight_row(ts, ty, rc.x0, rc.x1);
  return base[g] + local + (uint32_t)(tx - sp.x);
}

// Per-lane gradient terms of one splat for one pixel, back to front: consumes T (the
// transmittance behind the splat) and gS = g . S, returns them updated to the front of it.
// The nine terms are linear pieces of the splat's 2D gradient, finished once per workgroup:
//   v0 = s dx, v1 = s dy, v2 = s dx^2, v3 = s dx dy, v4 = s dy^2 (s = dL/dsigma), v5 = s,
//   v6..8 = alpha T_i g_rgb; then dL/dmean = (A P0 + B P1, B P0 + C P1), dL/dA = P2 / 2,
//   dL/dB = P3, dL/dC = P4 / 2, dL/do = -P5 / o (d alpha/do = G = alpha / o, d alpha/dsigma =
//   -alpha below the cap), dL/drgb = P6..8 (P = the sums over pixels).
// DEPTH: the depth channel is a fourth colour (value z, gradient gd): it joins g . c and g . S,
// and a tenth term v9 = alpha T_i gd gives dL/dz = P9.
template <bool DEPTH>
__device__ __forceinline__ void splat_grad(bool contrib, const SplatEval& ev, float dx, float dy, float cr, float cg,
                                           float cb, float z, float gr, float gg, float gb, float gd, float& T,
                                           float& gS, float* v) {
  const float inv = __builtin_amdgcn_rcpf(1.0f - ev.alpha);
  const float Ti = contrib ? T * inv : T;  // T_i, the transmittance in front of this splat
  const float gc = DEPTH ? fmaf(gd, z, fmaf(gr, cr, fmaf(gg, cg, gb * cb))) : fmaf(gr, cr, fmaf(gg, cg, gb * cb));
  const float g_alpha = fmaf(Ti, gc, -gS * inv);  // dL/dalpha = g . (c T_i - S / (1 - alpha))
  // alpha T_i as a product: Ti - T would save one operation but cancels for alpha near 1/255
  const float wT = contrib ? ev.alpha * Ti : 0.0f;
  gS = fmaf(gc, wT, gS);
  T = Ti;
  const float s = (contrib && !ev.capped) ? -ev.alpha * g_alpha : 0.0f;  // dL/dsigma
  const float p = s * dx, q = s * dy;
  v[0] = p;
  v[1] = q;
  v[2] = p * dx;
  v[3] = p * dy;
  v[4] = q * dy;
  v[5] = s;
  v[6] = wT * gr;
  v[7] = wT * gg;
  v[8] = wT * gb;
  if (DEPTH) v[9] = wT * gd;
}

// The per-splat sums of reduce9_to_lds, plus (DEPTH) the tenth term summed into acc[9].
// Two splats at once (a, b: nine terms each, summed over the wave into accA[0..8], accB[0..8]).
// A permlane32 swap + add first puts splat a's term j in the low half and b's in the high half;
// a permlane16 swap + add then leaves (a_k, a_k+4, b_k, b_k+4) in rows 0-3; a row_ror:8 exchange
// and a row_half_mirror exchange split each row into four 4-lane groups (k = 2 bit2 + bit3 of
// the lane), and two quad_perm adds finish each group: one register, 16 terms, fewer operations
// and independent chains for the scheduler. Term 8 of both: one swap, then row shifts and a
// row_bcast:15 leave a's sum in lane 31 and b's in lane 63.
template <bool STORE>
__device__ __forceinline__ void reduce18_to_lds(const float* a, const float* b, float* accA, float* accB, int lane) {
  float u[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = swap32_sum(a[j], b[j]);
  float w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = swap16_sum(u[k], u[k + 4]);  // rows: a_k, a_k+4, b_k, b_k+4
  const bool h8 = (lane & 8) != 0, h4 = (lane & 4) != 0;
  const float x01 = (h8 ? w[1] : w[0]) + dppx<0x128>(h8 ? w[0] : w[1]);  // row_ror:8: l <-> l ^ 8
  const float x23 = (h8 ? w[3] : w[2]) + dppx<0x128>(h8 ? w[2] : w[3]);
  float x = (h4 ? x23 : x01) + dppx<0x141>(h4 ? x01 : x23);  // row_half_mirror: l <-> 7 - l
  x = x + dppx<0x4E>(x);                                     // quad_perm [2,3,0,1]: l <-> l ^ 2
  x = x + dppx<0xB1>(x);                                     // quad_perm [1,0,3,2]: l <-> l ^ 1
  const int row = lane >> 4;
  const int term = (h4 ? 2 : 0) + (h8 ? 1 : 0) + ((row & 1) ? 4 : 0);
  float* acc = (row >> 1) ? accB : accA;
  const float y0 = swap32_sum(a[8], b[8]);  // a in lanes 0-31, b in lanes 32-63
  float y = y0 + dpp_f<0x111>(y0);          // row_shr:1
  y = y + dpp_f<0x112>(y0);                 // row_shr:2
  y = y + dpp_f<0x113>(y0);                 // row_shr:3
  y = y + dpp_f<0x114>(y);                  // row_shr:4
  y = y + dpp_f<0x118>(y);                  // row_shr:8: lane 15 of each row holds the row
  y = y + dpp_f<0x142>(y);                  // row_bcast:15: lane 31 rows 0 + 1, lane 63 rows 2 + 3
  float* acc8 = ((lane & 32) ? accB : accA) + 8;  // lanes 31 and 63 store, one instruction for both
  if (STORE) {
    if ((lane & 3) == 0) acc[term] = x;
    if ((lane & 31) == 31) *acc8 = y;
  } else {
    if ((lane & 3) == 0) unsafeAtomicAdd(acc + term, x);
    if ((lane & 31) == 31) unsafeAtomicAdd(acc8, y);
  }
}

template <bool STORE, bool DEPTH>
__device__ __forceinline__ void reduce_terms(const float* v, float* acc, int lane) {
  reduce9_to_lds<STORE>(v, acc, lane);
  if (DEPTH) {
    const float y = wave_sum_lane63(v[9]);
    if (lane == 63) {
      if (STORE)
        acc[9] = y;
      else
        unsafeAtomicAdd(acc + 9, y);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// k-rbwd: same tiling; each wave walks its quadrant's splats back to front from the last
// contributor of its pixels, recovering T_i = T_{i+1} / (1 - alpha_i), two splats per
// iteration (their alphas are independent; only the T / g.S updates are sequential).
// With a raster plan and the forward's checkpoints, workgroup b takes work item b: one chunk
// [c L, (c + 1) L) of a tile's list. An inner chunk starts from the transmittance stored after
// it and from S = T_final background + the colour that every later chunk added (summed back to
// front, like the sums of the whole-tile walk: a sum of the terms, never a difference).
// Where the 2D gradient of a (tile, splat) pair goes (MODE):
//   kBwdAtomic  added to g2d [9, n] with global fp32 atomics;
//   kBwdDeterministic  written to its own slot of rec [rec_cap, 10] (pair_slot), summed per
//               Gaussian later in a fixed order; the four waves' sums of a splat are kept apart in
//               LDS (per 64-splat group, with a barrier after each group) and added in wave order,
//               so every floating-point sum has a fixed order: bitwise-reproducible gradients
//               (LDS atomics across the waves instead of the barriers measured slower).
// With records, the slots of the pairs a chunk does not stage (behind every pixel's last
// contributor) get zeros, so that all P records are written by the launch.
// ---------------------------------------------------------------------------------------------
constexpr int kBwdAtomic = 0, kBwdDeterministic = 2;
constexpr int kG2d = 10;  // components of a 2D gradient: mean2d (2), conic (3), opacity, rgb (3), depth
// DEPTH: the backward of the depth channel too (dL/ddepth given; tenth component dL/dz).
template <bool COUNT, int MODE, bool DEPTH>
__global__ __launch_bounds__(kRasterThreads) __attribute__((amdgpu_waves_per_eu(7))) void k_rbwd(
    uint32_t n, const uint32_t* __restrict__ ranges, const uint32_t* __restrict__ plan, uint32_t ntiles,
    const float4* __restrict__ ckpt, const float* __restrict__ ckpt_d, const uint32_t* __restrict__ ids,
    const float* __restrict__ means2d, const float* __restrict__ conics, const float* __restrict__ opac,
    const float* __restrict__ colors, const float* __restrict__ depths, const int32_t* __restrict__ radii,
    DevCamera cam, const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib,
    const float* __restrict__ dL_dimage, const float* __restrict__ dL_ddepth, float* __restrict__ g2d,
    const uint32_t* __restrict__ pair_base, float* __restrict__ rec, uint32_t rec_cap,
    unsigned long long* __restrict__ eval_count) {
  // g2d is [10, n]: component c of splat g at c * n + g; rec is [rec_cap, 10] (a pair's 40 B
  // together); without DEPTH the tenth component is not written (it stays 0)
  constexpr bool REC = MODE != kBwdAtomic, DET = MODE == kBwdDeterministic;
  constexpr int NT = DEPTH ? 10 : 9;  // terms summed per splat
  using BZ = typename std::conditional<DEPTH, float2, float4>::type;
  __shared__ float4 s_a[kBatch];
  __shared__ float4 s_b[kBatch];
  __shared__ BZ s_c[kBatch];
  __shared__ uint32_t s_id[kBatch];
  __shared__ float s_acc[(kBatch + (DEPTH ? 0 : 4)) * NT];  // the splats' sums (then a spare slot per wave)
  __shared__ uint64_t s_qm[4][4];
  __shared__ uint32_t s_max;

  // the work: a whole tile (no checkpoints) or one chunk of a tile's list
  int tile;
  uint32_t lo = 0, hi = 0xFFFFFFFFu, chunk = 0, nch = 0;
  bool from_ckpt = false;
  size_t slot0 = 0;
  if (plan && ckpt) {
    // work items: the extra ones (chunks >= 1 of long tiles), then chunk 0 of every tile in order
    const uint32_t nx = plan[kPlanExtra];
    if (blockIdx.x < nx) {
      const uint32_t* item = plan + kPlanOrder + 2 * ntiles + 2 * blockIdx.x;
      tile = (int)item[0];
      chunk = item[1];
    } else {
      // the tiles from a multiple of 8 on: order slot i runs on XCD i mod 8
      const uint32_t b0 = plan_xcd_align(nx);
      if (blockIdx.x < b0 || blockIdx.x - b0 >= ntiles) return;  // workgroup-uniform
      tile = (int)plan[kPlanOrder + blockIdx.x - b0];
    }
    const uint32_t L = plan[kPlanChunk];
    const uint32_t len = ranges[2 * tile + 1] - ranges[2 * tile];
    nch = (len + L - 1) / L;
    lo = chunk * L;
    hi = lo + L;
    if (hi < len) {
      from_ckpt = true;
      slot0 = (size_t)plan[kPlanOrder + ntiles + tile] * kRasterThreads;
    }
  } else {
    tile = plan ? (int)plan[kPlanOrder + blockIdx.x] : (int)blockIdx.x;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
  const float tx0 = (float)(tx * kTile), ty0 = (float)(ty * kTile);
  const int px_i = tx * kTile + (wave & 1) * 8 + (lane & 7);
  const int py_i = ty * kTile + (wave >> 1) * 8 + (lane >> 3);
  const bool inside = px_i < cam.W && py_i < cam.H;
  const float px = (float)px_i + 0.5f, py = (float)py_i + 0.5f;
  const uint32_t start = ranges[2 * tile];
  const uint32_t len = ranges[2 * tile + 1] - start;
  const uint32_t chunk_end = hi < len ? hi : len;

  // Stage splats [bstart, bstart + cnt) of the list: ids, evaluation records and quadrant masks in
  // LDS, the sums zeroed; with records, the staging thread keeps its splat's record slot.
  uint32_t rslot = 0;
  auto stage = [&](uint32_t bstart, int cnt) {
    uint32_t qm = 0;
    if (tid < cnt) {
      const uint32_t g = ids[start + bstart + (uint32_t)tid];
      s_id[tid] = g;
      const RawSplat rs = load_raw<DEPTH>(g, n, means2d, conics, opac, colors, depths);
      qm = stage_raw(rs, g < n, tx0, ty0, s_a[tid], s_b[tid], s_c[tid]);
      if (REC && g < n) rslot = pair_slot(g, means2d, radii, pair_base, tx, ty, cam, rs.A, rs.B, rs.C, rs.o);
    }
    if (!DET)
      for (int i = tid; i < cnt * NT; i += kRasterThreads) s_acc[i] = 0.0f;
    publish_quadrant_masks(qm, tid < cnt, s_qm);
  };
  // the 2D gradient of staged splat tid from its sums P, to g2d or its record slot
  // The conic is taken back from the staged record (its log2(e) scaling undone: within an ulp of
  // the raw conic), the opacity as staged; so nothing of the splat stays in registers through the walk.
  auto finish = [&](const float* P) {
    const uint32_t g = s_id[tid];
    const float4 ra = s_a[tid], rb = s_b[tid];
    const float A = ra.z / (0.5f * kLog2e), B = rb.x / kLog2e, C = ra.w / (0.5f * kLog2e), o = rb.y;
    float gv[kG2d];
    gv[0] = fmaf(A, P[0], B * P[1]);
    gv[1] = fmaf(B, P[0], C * P[1]);
    gv[2] = 0.5f * P[2];
    gv[3] = P[3];
    gv[4] = 0.5f * P[4];
    gv[5] = -P[5] / o;
    gv[6] = P[6];
    gv[7] = P[7];
    gv[8] = P[8];
    gv[9] = DEPTH ? P[9] : 0.0f;
    if (REC) {
      if (rslot < rec_cap) {  // every component (without DEPTH the tenth is 0)
#pragma unroll
        for (int c = 0; c < kG2d; ++c) rec[(size_t)rslot * kG2d + c] = gv[c];
      }
    } else {
      // one plane per component: the atomics of a lane go to different cache lines
#pragma unroll
      for (int c = 0; c < NT; ++c)
        if (gv[c] != 0.0f) unsafeAtomicAdd(g2d + (size_t)c * n + g, gv[c]);
    }
  };
  const bool single = chunk_end <= lo + (uint32_t)kBatch;

  float T = 1.0f, gr = 0.0f, gg = 0.0f, gb = 0.0f, gd = 0.0f, gS = 0.0f;
  uint32_t nc = 0;
  if (inside) {
    const int p = py_i * cam.W + px_i;
    nc = n_contrib[p];
    gr = dL_dimage[3 * p];
    gg = dL_dimage[3 * p + 1];
    gb = dL_dimage[3 * p + 2];
    if (DEPTH) gd = dL_ddepth[p];
    if (from_ckpt) {
      // S after the chunk = T_final background + the colour of chunks nch - 1 .. chunk + 1
      // (the depth channel: the later chunks' depth, background depth 0)
      const float Tf = final_T[p];
      float sr = Tf * cam.bg[0], sg = Tf * cam.bg[1], sb = Tf * cam.bg[2], sd = 0.0f;
      for (uint32_t k = nch - 1; k > chunk; --k) {
        const float4 st = ckpt[slot0 + (size_t)k * kRasterThreads + tid];
        sr += st.y;
        sg += st.z;
        sb += st.w;
        if (DEPTH) sd += ckpt_d[slot0 + (size_t)k * kRasterThreads + tid];
      }
      T = ckpt[slot0 + (size_t)chunk * kRasterThreads + tid].x;
      gS = (gr * sr + gg * sg) + gb * sb;
      if (DEPTH) gS = fmaf(gd, sd, gS);
    } else {
      // g . S with S = T_final background
      T = final_T[p];
      gS = T * ((gr * cam.bg[0] + gg * cam.bg[1]) + gb * cam.bg[2]);
    }
  }
  // a chunk of at most one batch is staged at once, after the pixels' loads above are issued,
  // so that its own chain of loads (ids, then records) overlaps them
  if (single && chunk_end > lo) stage(lo, (int)(chunk_end - lo));
  if (tid == 0) s_max = 0;
  __syncthreads();
  const uint32_t wmax = wave_max_lane63(nc);
  if (lane == 63 && wmax) atomicMax(&s_max, wmax);
  __syncthreads();
  const uint32_t max_nc = s_max < hi ? s_max : hi;
  uint32_t n_eval = 0;
  if (REC && !single) {
    // the pairs behind every pixel's last contributor are never staged: their records get
    // zeros here, so that every record of the P pairs is written once (a single batch stages
    // its whole chunk, and the walk's batches cover [lo, max_nc))
    for (uint32_t e = (max_nc > lo ? max_nc : lo) + (uint32_t)tid; e < chunk_end; e += kRasterThreads) {
      const uint32_t g = ids[start + e];
      if (g >= n) continue;
      const bool tt = cam.tight_tiles != 0;
      const uint32_t zs = pair_slot(g, means2d, radii, pair_base, tx, ty, cam, tt ? conics[3 * g] : 1.0f,
                                    tt ? conics[3 * g + 1] : 0.0f, tt ? conics[3 * g + 2] : 1.0f, tt ? opac[g] : 0.0f);
      if (zs < rec_cap) {
#pragma unroll
        for (int c = 0; c < kG2d; ++c) rec[(size_t)zs * kG2d + c] = 0.0f;
      }
    }
  }

  // a staged single batch covers [lo, chunk_end), which holds [lo, max_nc)
  for (uint32_t bend = single ? chunk_end : max_nc; bend > lo;) {
    const uint32_t bstart = bend > lo + (uint32_t)kBatch ? bend - kBatch : lo;
    const int cnt = (int)(bend - bstart);
    if (!single) {
      __syncthreads();
      stage(bstart, cnt);
    }
    __syncthreads();
    for (int w = 3; w >= 0; --w) {
      if (w * 64 >= cnt) continue;  // workgroup-uniform: no splat staged in this group
      // DET: this wave's sums of group w's 64 splats, zeroed first (row `lane` per lane)
      float* part = s_acc + (size_t)wave * 64 * NT;
      if (DET) {
#pragma unroll
        for (int c = 0; c < NT; ++c) part[lane * NT + c] = 0.0f;
      }
      uint64_t m = uniform64(s_qm[wave][w]);  // walked from the highest set bit down
      while (m) {
        const int bit0 = 63 - __builtin_clzll(m);
        m ^= 1ull << bit0;
        const bool has1 = m != 0;
        const int bit1 = has1 ? 63 - __builtin_clzll(m) : bit0;
        m &= ~(1ull << bit1);  // no-op when !has1 (m is already 0)
        const int k0 = __builtin_amdgcn_readfirstlane(w * 64 + bit0);
        const int k1 = __builtin_amdgcn_readfirstlane(w * 64 + bit1);
        // the lanes that have reached each splat (from their last contributor back)
        const uint64_t act0_m = lanes_where(bstart + (uint32_t)k0 < nc);
        const uint64_t act1_m = has1 ? lanes_where(bstart + (uint32_t)k1 < nc) : 0ull;
        if ((act0_m | act1_m) == 0ull) continue;
        const bool act0 = lane_in(act0_m), act1 = lane_in(act1_m);
        const float4 a0 = s_a[k0], b0 = s_b[k0];
        const float4 a1 = s_a[k1], b1 = s_b[k1];
        const float2 cz0 = *reinterpret_cast<const float2*>(&s_c[k0]);
        const float2 cz1 = *reinterpret_cast<const float2*>(&s_c[k1]);
        const float cb0 = cz0.x, cb1 = cz1.x;
        const float z0 = DEPTH ? cz0.y : 0.0f, z1 = DEPTH ? cz1.y : 0.0f;
        const float dx0 = a0.x - px, dy0 = a0.y - py, dx1 = a1.x - px, dy1 = a1.y - py;
        const SplatEval e0 = eval_splat(dx0, dy0, a0.z, b0.x, a0.w, b0.y);
        const SplatEval e1 = eval_splat(dx1, dy1, a1.z, b1.x, a1.w, b1.y);
        if (COUNT) n_eval += (act0 ? 1u : 0u) + (act1 ? 1u : 0u);
        const uint64_t c0_m = act0_m & ~lanes_skipped(e0), c1_m = act1_m & ~lanes_skipped(e1);
        const bool c0 = lane_in(c0_m), c1 = lane_in(c1_m);
        float v0[NT], v1[NT];
        splat_grad<DEPTH>(c0, e0, dx0, dy0, b0.z, b0.w, cb0, z0, gr, gg, gb, gd, T, gS, v0);
        splat_grad<DEPTH>(c1, e1, dx1, dy1, b1.z, b1.w, cb1, z1, gr, gg, gb, gd, T, gS, v1);
        float* acc0 = DET ? part + (k0 - w * 64) * NT : s_acc + k0 * NT;
        float* acc1 = !has1 ? (DEPTH ? acc0 : s_acc + (kBatch + wave) * NT)  // (DEPTH: never used)
                            : DET ? part + (k1 - w * 64) * NT : s_acc + k1 * NT;
        if (!DEPTH) {
          // both splats in one reduction: a splat no lane reaches adds zeros to its own slot, and
          // the missing partner of a lone splat (its terms all zero) goes to the wave's spare slot,
          // which is never read; one path, so the compiler keeps no copies of the terms
          if ((c0_m | c1_m) != 0ull) reduce18_to_lds<DET>(v0, v1, acc0, acc1, lane);
        } else {
          if (c0_m != 0ull) reduce_terms<DET, DEPTH>(v0, acc0, lane);
          if (c1_m != 0ull) reduce_terms<DET, DEPTH>(v1, acc1, lane);
        }
      }
      if (DET) {
        // group w is staged by wave w: its threads add the four waves' sums in wave order
        __syncthreads();
        if (wave == w && tid < cnt && s_id[tid] < n) {
          float P[NT];
#pragma unroll
          for (int c = 0; c < NT; ++c) {
            float acc = s_acc[(0 * 64 + lane) * NT + c];
            acc += s_acc[(1 * 64 + lane) * NT + c];
            acc += s_acc[(2 * 64 + lane) * NT + c];
            acc += s_acc[(3 * 64 + lane) * NT + c];
            P[c] = acc;
          }
          finish(P);
        }
        __syncthreads();
      }
    }
    __syncthreads();
    // finish the 2D gradient of each staged splat from its nine sums
    if (!DET && tid < cnt && s_id[tid] < n) finish(s_acc + tid * NT);
    bend = bstart;
  }
  if (COUNT) count_evals(n_eval, eval_count);
}

// dL/d(2D parameters) of Gaussian g from its records, in an order fixed by its pair count. A
// wave takes 64 consecutive Gaussians, one per lane (every lane of the wave calls this; g may be
// past n): a lane whose Gaussian has at most kSegLane pairs adds its records in slot order (a
// record is 40 B, read as five float2). The Gaussians of more pairs are then taken one at a time
// by the whole wave: lane l adds records l, l + 64, ... in order and a fixed DPP tree adds the
// lanes. When the pairs did not fit the records (fits false: the pair sort then left every tile
// range empty) every gradient is zero.
constexpr uint32_t kSegLane = 16;
__device__ __forceinline__ void seg_sum(int32_t n, int64_t g, int lane, const uint32_t* __restrict__ tiles_touched,
                                        const uint32_t* __restrict__ base, bool fits, const float* __restrict__ rec,
                                        float* acc) {
  const uint32_t cnt = (g < n && fits) ? tiles_touched[g] : 0u;
  const uint32_t b = g < n ? base[g] : 0u;
#pragma unroll
  for (int c = 0; c < kG2d; ++c) acc[c] = 0.0f;
  if (cnt <= kSegLane) {
    // four records in flight at a time, added in slot order (a missing one adds nothing)
    for (uint32_t j = 0; j < cnt; j += 4) {
      float2 v[4][kG2d / 2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2* r = reinterpret_cast<const float2*>(rec + ((size_t)b + j + (uint32_t)i) * kG2d);
#pragma unroll
        for (int c = 0; c < kG2d / 2; ++c) v[i][c] = j + (uint32_t)i < cnt ? r[c] : make_float2(0.0f, 0.0f);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j + (uint32_t)i < cnt) {
#pragma unroll
          for (int c = 0; c < kG2d / 2; ++c) {
            acc[2 * c] += v[i][c].x;
            acc[2 * c + 1] += v[i][c].y;
          }
        }
      }
    }
  }
  uint64_t big = __ballot(cnt > kSegLane);
  while (big) {
    const int src = __builtin_ctzll(big);
    big &= big - 1;
    const uint32_t cb = __builtin_amdgcn_readlane(cnt, src), bb = __builtin_amdgcn_readlane(b, src);
    float w[kG2d];
#pragma unroll
    for (int c = 0; c < kG2d; ++c) w[c] = 0.0f;
    for (uint32_t j = lane; j < cb; j += 64) {
#pragma unroll
      for (int c = 0; c < kG2d; ++c) w[c] += rec[((size_t)bb + j) * kG2d + c];
    }
#pragma unroll
    for (int c = 0; c < kG2d; ++c) {
      const float t = wave_sum_lane63(w[c]);
      const float tb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 63));
      if (lane == src) acc[c] = tb;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// k-pbwd: chain rule from the 2D gradients (mean2d, conic, opacity, colour) to the raw
// parameters (sections 1-4 of the PyTorch lesson, differentiated). One thread per Gaussian.
// The decisions (culled, J clamps, det clamp) are the forward's: the fp32 projection is replayed
// bit for bit. The chain itself runs in fp64: it is O(N) work, and in fp32 it loses up to three
// digits for needle-like splats (inverting a near-singular 2x2) and for SH terms that cancel.
// Scale and rotation gradients go through Q = J W R (2x3): Sigma' - 0.3 I = sum_j s_j^2 q_j q_j^T,
// so dL/dl_j = 2 s_j^2 q_j^T G2 q_j, dL/dQ = 2 G2 Q S^2 and dL/dR = (J W)^T dL/dQ.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void sh_basis_grad_f64(int degree, double x, double y, double z, double* B,
                                                  double (*dB)[3]) {
  const double s3 = 1.7320508075688772, s15 = 3.872983346207417, s5 = 2.23606797749979,
               s15h = 1.9364916731037085, s358 = 2.091650066335189, s105 = 10.246950765959598,
               s218 = 1.6201851746019651, s7h = 1.3228756555322954, s105h = 5.123475382979799,
               s5h = 1.118033988749895;
  for (int k = 0; k < 16; ++k) dB[k][0] = dB[k][1] = dB[k][2] = 0.0;
  B[0] = 1.0;
  if (degree < 1) return;
  B[1] = s3 * y; dB[1][1] = s3;
  B[2] = s3 * z; dB[2][2] = s3;
  B[3] = s3 * x; dB[3][0] = s3;
  if (degree < 2) return;
  B[4] = s15 * x * y; dB[4][0] = s15 * y; dB[4][1] = s15 * x;
  B[5] = s15 * y * z; dB[5][1] = s15 * z; dB[5][2] = s15 * y;
  B[6] = s5h * (3.0 * z * z - 1.0); dB[6][2] = 3.0 * s5 * z;
  B[7] = s15 * x * z; dB[7][0] = s15 * z; dB[7][2] = s15 * x;
  B[8] = s15h * (x * x - y * y); dB[8][0] = s15 * x; dB[8][1] = -s15 * y;
  if (degree < 3) return;
  B[9] = s358 * y * (3.0 * x * x - y * y);
  dB[9][0] = 6.0 * s358 * x * y; dB[9][1] = 3.0 * s358 * (x * x - y * y);
  B[10] = s105 * x * y * z;
  dB[10][0] = s105 * y * z; dB[10][1] = s105 * x * z; dB[10][2] = s105 * x * y;
  B[11] = s218 * y * (5.0 * z * z - 1.0);
  dB[11][1] = s218 * (5.0 * z * z - 1.0); dB[11][2] = 10.0 * s218 * y * z;
  B[12] = s7h * z * (5.0 * z * z - 3.0);
  dB[12][2] = s7h * (15.0 * z * z - 3.0);
  B[13] = s218 * x * (5.0 * z * z - 1.0);
  dB[13][0] = s218 * (5.0 * z * z - 1.0); dB[13][2] = 10.0 * s218 * x * z;
  B[14] = s105h * z * (x * x - y * y);
  dB[14][0] = 2.0 * s105h * x * z; dB[14][1] = -2.0 * s105h * y * z; dB[14][2] = s105h * (x * x - y * y);
  B[15] = s358 * x * (x * x - 3.0 * y * y);
  dB[15][0] = 3.0 * s358 * (x * x - y * y); dB[15][1] = -6.0 * s358 * x * y;
}

// SEG (the deterministic backward): the 2D gradient is summed from the per-pair records here
// (seg_sum: a wave per 64 consecutive Gaussians, the same lanes as the chain rule's), else read
// from g2d [10, n].
template <int DEG, bool SEG>
__global__ __launch_bounds__(256) void k_pbwd(
    int32_t n, const float* __restrict__ means, const float* __restrict__ log_scales, const float* __restrict__ quats,
    const float* __restrict__ logits, const float* __restrict__ sh, DevCamera cam,
    const uint32_t* __restrict__ tiles_touched, const float* __restrict__ g2d, const uint32_t* __restrict__ base,
    const unsigned long long* __restrict__ total, const float* __restrict__ rec, uint32_t rec_cap,
    float* __restrict__ d_means, float* __restrict__ d_log_scales, float* __restrict__ d_quats,
    float* __restrict__ d_logits, float* __restrict__ d_sh, float* __restrict__ d_means2d) {
  constexpr int K = (DEG + 1) * (DEG + 1);
  const int g = blockIdx.x * 256 + threadIdx.x;
  double G9[kG2d];  // the 2D gradient; G9[9] is dL/d(camera z) of the depth channel
  if (SEG) {
    if (blockIdx.x * 256 + (threadIdx.x & ~63) >= n) return;  // wave-uniform: the wave's first Gaussian
    float acc[kG2d];
    seg_sum(n, g, threadIdx.x & 63, tiles_touched, base, *total <= (unsigned long long)rec_cap, rec, acc);
    if (g >= n) return;
#pragma unroll
    for (int c = 0; c < kG2d; ++c) G9[c] = (double)acc[c];
  } else {
    if (g >= n) return;
#pragma unroll
    for (int c = 0; c < kG2d; ++c) G9[c] = (double)g2d[(size_t)c * n + g];  // [10, n]
  }
  double gm[3] = {0, 0, 0}, gl[3] = {0, 0, 0}, gq4[4] = {0, 0, 0, 0}, glogit = 0.0;
  double gsh[K * 3];
#pragma unroll
  for (int i = 0; i < K * 3; ++i) gsh[i] = 0.0;

  const bool drawn = tiles_touched[g] > 0;
  if (drawn) {
    const float m0f = means[3 * g], m1f = means[3 * g + 1], m2f = means[3 * g + 2];
    const float l0f = log_scales[3 * g], l1f = log_scales[3 * g + 1], l2f = log_scales[3 * g + 2];
    const float4 q4 = *reinterpret_cast<const float4*>(quats + 4 * g);
    const float logitf = logits[g];
    float shc[K * 3];
#pragma unroll
    for (int i = 0; i < K * 3; ++i) shc[i] = sh[(size_t)g * (K * 3) + i];
    // the forward's decisions
    const ProjF32 P32 = project_f32<DEG, false>(m0f, m1f, m2f, l0f, l1f, l2f, q4, logitf, shc, cam);

    // ---- forward intermediates in fp64 ----
    const double mu[3] = {m0f, m1f, m2f};
    const double qw = q4.x, qx = q4.y, qy = q4.z, qz = q4.w;
    const double qn_raw = sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
    const double qn = qn_raw > 1e-12 ? qn_raw : 1e-12;
    const double w = qw / qn, x = qx / qn, y = qy / qn, z = qz / qn;
    const double s[3] = {exp((double)l0f), exp((double)l1f), exp((double)l2f)};
    const double o = 1.0 / (1.0 + exp(-(double)logitf));
    double R[9];
    R[0] = 1.0 - 2.0 * (y * y + z * z);
    R[1] = 2.0 * (x * y - w * z);
    R[2] = 2.0 * (x * z + w * y);
    R[3] = 2.0 * (x * y + w * z);
    R[4] = 1.0 - 2.0 * (x * x + z * z);
    R[5] = 2.0 * (y * z - w * x);
    R[6] = 2.0 * (x * z - w * y);
    R[7] = 2.0 * (y * z + w * x);
    R[8] = 1.0 - 2.0 * (x * x + y * y);
    double W[9], w0[3];
    for (int r = 0; r < 3; ++r) {
      for (int c = 0; c < 3; ++c) W[r * 3 + c] = (double)cam.V[r * 4 + c];
      w0[r] = (double)cam.V[r * 4 + 3];
    }
    double t[3];
    for (int r = 0; r < 3; ++r) t[r] = W[r * 3] * mu[0] + W[r * 3 + 1] * mu[1] + W[r * 3 + 2] * mu[2] + w0[r];
    const double tx = t[0], ty = t[1], tz = t[2];
    const double fx = cam.fx, fy = cam.fy, cx = cam.cx, cy = cam.cy;
    const double tfx = 0.5 * (double)cam.W / fx, tfy = 0.5 * (double)cam.H / fy;
    const double lxl = -(cx / fx + 0.3 * tfx), lxh = ((double)cam.W - cx) / fx + 0.3 * tfx;
    const double lyl = -(cy / fy + 0.3 * tfy), lyh = ((double)cam.H - cy) / fy + 0.3 * tfy;
    const double xz = tx / tz, yz = ty / tz;
    const double jx = tz * fmin(fmax(xz, lxl), lxh), jy = tz * fmin(fmax(yz, lyl), lyh);
    const double iz = 1.0 / tz, iz2 = iz * iz;
    const double J[6] = {fx * iz, 0.0, -fx * jx * iz2, 0.0, fy * iz, -fy * jy * iz2};
    double JW[6], Q[6];
    for (int a2 = 0; a2 < 2; ++a2)
      for (int j = 0; j < 3; ++j) JW[a2 * 3 + j] = J[a2 * 3] * W[j] + J[a2 * 3 + 1] * W[3 + j] + J[a2 * 3 + 2] * W[6 + j];
    for (int a2 = 0; a2 < 2; ++a2)
      for (int j = 0; j < 3; ++j) Q[a2 * 3 + j] = JW[a2 * 3] * R[j] + JW[a2 * 3 + 1] * R[3 + j] + JW[a2 * 3 + 2] * R[6 + j];
    double a0 = 0.0, b = 0.0, c0 = 0.0;  // Sigma2d before the dilation
    for (int j = 0; j < 3; ++j) {
      const double s2 = s[j] * s[j];
      a0 += s2 * Q[j] * Q[j];
      b += s2 * Q[j] * Q[3 + j];
      c0 += s2 * Q[3 + j] * Q[3 + j];
    }
    const double a = a0 + 0.3, c = c0 + 0.3;
    // Sigma_c = W Sigma W^T = (W R) S^2 (W R)^T, for J's dependence on t
    double WR[9], Sc[9];
    for (int i = 0; i < 3; ++i)
      for (int j = 0; j < 3; ++j) WR[i * 3 + j] = W[i * 3] * R[j] + W[i * 3 + 1] * R[3 + j] + W[i * 3 + 2] * R[6 + j];
    for (int i = 0; i < 3; ++i)
      for (int k = 0; k < 3; ++k)
        Sc[i * 3 + k] = s[0] * s[0] * WR[i * 3] * WR[k * 3] + s[1] * s[1] * WR[i * 3 + 1] * WR[k * 3 + 1] +
                        s[2] * s[2] * WR[i * 3 + 2] * WR[k * 3 + 2];

    // ---- conic (A, B, C) = (c, -b, a) / det  ->  dL/d(a, b, c) ----
    const double gA = G9[2], gB = G9[3], gC = G9[4];
    double ga, gb, gc;
    if (!P32.det_clamped) {
      const double id = 1.0 / (a * c - b * b);
      const double PA = c * id, PB = -b * id, PC = a * id;
      ga = -(gA * PA * PA + gB * PA * PB + gC * PB * PB);
      gc = -(gA * PB * PB + gB * PB * PC + gC * PC * PC);
      gb = -2.0 * (gA * PA * PB + 0.5 * gB * (PA * PC + PB * PB) + gC * PB * PC);
    } else {
      ga = gC * 1e10;
      gb = -gB * 1e10;
      gc = gA * 1e10;
    }
    // ---- antialiased opacity o comp, comp = sqrt(det0 / det): d comp = comp / 2 (d det0 / det0 -
    // d det / det), det0 = a0 c0 - b^2, det = a c - b^2, da = da0, dc = dc0 ----
    double comp = 1.0;
    if (cam.antialiased) {
      const double det0 = a0 * c0 - b * b, det1 = a * c - b * b;
      comp = det0 > 0.0 ? sqrt(det0 / det1) : 0.0;
      if (comp > 0.0) {
        const double h = 0.5 * G9[5] * o * comp;
        ga += h * (c0 / det0 - c / det1);
        gc += h * (a0 / det0 - a / det1);
        gb += h * (2.0 * b / det1 - 2.0 * b / det0);
      }
    }
    const double G2[4] = {ga, 0.5 * gb, 0.5 * gb, gc};

    // ---- scales and rotation through Q ----
    double gR[9];
    for (int j = 0; j < 3; ++j) {
      const double q0 = Q[j], q1 = Q[3 + j];
      const double u0 = G2[0] * q0 + G2[1] * q1, u1 = G2[2] * q0 + G2[3] * q1;
      const double s2 = s[j] * s[j];
      gl[j] = 2.0 * s2 * (q0 * u0 + q1 * u1);
      const double gQ0 = 2.0 * s2 * u0, gQ1 = 2.0 * s2 * u1;
      for (int i = 0; i < 3; ++i) gR[i * 3 + j] = JW[i] * gQ0 + JW[3 + i] * gQ1;
    }
    gq4[0] = 2.0 * (-z * gR[1] + y * gR[2] + z * gR[3] - x * gR[5] - y * gR[6] + x * gR[7]);
    gq4[1] = 2.0 * (y * gR[1] + z * gR[2] + y * gR[3] - 2.0 * x * gR[4] - w * gR[5] + z * gR[6] + w * gR[7] -
                    2.0 * x * gR[8]);
    gq4[2] = 2.0 * (-2.0 * y * gR[0] + x * gR[1] + w * gR[2] + x * gR[3] + z * gR[5] - w * gR[6] + z * gR[7] -
                    2.0 * y * gR[8]);
    gq4[3] = 2.0 * (-2.0 * z * gR[0] - w * gR[1] + x * gR[2] + w * gR[3] - 2.0 * z * gR[4] + y * gR[5] +
                    x * gR[6] + y * gR[7]);
    {
      const double qh[4] = {w, x, y, z};
      if (qn_raw > 1e-12) {
        const double dot = w * gq4[0] + x * gq4[1] + y * gq4[2] + z * gq4[3];
        for (int j = 0; j < 4; ++j) gq4[j] = (gq4[j] - qh[j] * dot) / qn;
      } else {
        for (int j = 0; j < 4; ++j) gq4[j] = gq4[j] / qn;
      }
    }

    // ---- the camera-space mean: through J (dL/dJ = 2 G2 J Sc) and through mean2d ----
    double GJ[6];
    for (int p2 = 0; p2 < 2; ++p2)
      for (int j = 0; j < 3; ++j) GJ[p2 * 3 + j] = G2[p2 * 2] * J[j] + G2[p2 * 2 + 1] * J[3 + j];
    double gJ[6];
    for (int p2 = 0; p2 < 2; ++p2)
      for (int j = 0; j < 3; ++j)
        gJ[p2 * 3 + j] = 2.0 * (GJ[p2 * 3] * Sc[j] + GJ[p2 * 3 + 1] * Sc[3 + j] + GJ[p2 * 3 + 2] * Sc[6 + j]);
    double gt[3] = {0.0, 0.0, 0.0};
    gt[2] -= (gJ[0] * fx + gJ[4] * fy) * iz2;
    {
      const double dxx = P32.clamp_x ? 0.0 : 1.0, dxz = P32.clamp_x ? jx * iz : 0.0;
      gt[0] += gJ[2] * (-fx * iz2) * dxx;
      gt[2] += gJ[2] * (2.0 * fx * jx * iz2 * iz - fx * dxz * iz2);
      const double dyy = P32.clamp_y ? 0.0 : 1.0, dyz = P32.clamp_y ? jy * iz : 0.0;
      gt[1] += gJ[5] * (-fy * iz2) * dyy;
      gt[2] += gJ[5] * (2.0 * fy * jy * iz2 * iz - fy * dyz * iz2);
    }
    gt[0] += G9[0] * fx * iz;
    gt[2] -= G9[0] * fx * tx * iz2;
    gt[1] += G9[1] * fy * iz;
    gt[2] -= G9[1] * fy * ty * iz2;
    gt[2] += G9[9];  // the depth channel's value is t_z
    for (int j = 0; j < 3; ++j) gm[j] = W[j] * gt[0] + W[3 + j] * gt[1] + W[6 + j] * gt[2];

    // ---- log-scales, opacity, colour ----
    glogit = o * (1.0 - o) * comp * G9[5];
    if (DEG == 0) {
      gsh[0] = G9[6]; gsh[1] = G9[7]; gsh[2] = G9[8];
    } else {
      double C[3];
      for (int j = 0; j < 3; ++j) C[j] = -(W[j] * w0[0] + W[3 + j] * w0[1] + W[6 + j] * w0[2]);
      const double d[3] = {mu[0] - C[0], mu[1] - C[1], mu[2] - C[2]};
      const double dnr = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
      const double dn = dnr > 1e-12 ? dnr : 1e-12;
      const double u[3] = {d[0] / dn, d[1] / dn, d[2] / dn};
      double B[16], dB[16][3];
      sh_basis_grad_f64(DEG, u[0], u[1], u[2], B, dB);
      double gd[3] = {0.0, 0.0, 0.0};
#pragma unroll
      for (int l = 0; l < K; ++l)
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
          gsh[l * 3 + ch] = B[l] * G9[6 + ch];
          if (l > 0) {
            const double wgt = (double)shc[l * 3 + ch] * G9[6 + ch];
            for (int j = 0; j < 3; ++j) gd[j] += wgt * dB[l][j];
          }
        }
      const double dot = u[0] * gd[0] + u[1] * gd[1] + u[2] * gd[2];
      for (int j = 0; j < 3; ++j) gm[j] += (gd[j] - u[j] * dot) / dn;
    }
  }
  for (int j = 0; j < 3; ++j) d_means[3 * g + j] = (float)gm[j];
  for (int j = 0; j < 3; ++j) d_log_scales[3 * g + j] = (float)gl[j];
  *reinterpret_cast<float4*>(d_quats + 4 * g) = make_float4((float)gq4[0], (float)gq4[1], (float)gq4[2], (float)gq4[3]);
  d_logits[g] = (float)glogit;
#pragma unroll
  for (int i = 0; i < K * 3; ++i) d_sh[(size_t)g * (K * 3) + i] = (float)gsh[i];
  if (d_means2d) {
    d_means2d[2 * g] = drawn ? (float)G9[0] : 0.0f;
    d_means2d[2 * g + 1] = drawn ? (float)G9[1] : 0.0f;
  }
}

__global__ void k_fill_zero(float* __restrict__ p, size_t count) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// Clears the records of the P = *total pairs (none when P exceeds the capacity: nothing is then
// read), four floats per store.

// ---------------------------------------------------------------------------------------------
// Per-pair records: base[g] = sum of tiles_touched over ids < g (exclusive prefix in id order),
// total = the sum over all ids (= P). Two launches, reduce then scan, over blocks of 4096 ids;
// integer sums, so the result does not depend on the order of the additions. Up to kBaseOne
// blocks the scan launch alone does it, each block summing the counts of all ids before it (at
// most 15 x 4096, eight loads in flight per thread). The records need no clearing: the backward
// writes every pair's record, zeros for the pairs it does not stage.
// ---------------------------------------------------------------------------------------------
constexpr int kBaseThreads = 1024, kBaseItems = 4, kBaseTile = kBaseThreads * kBaseItems;
constexpr unsigned kBaseOne = 16;

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* s_w) {
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_w[wave] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < kBaseThreads / 64; ++w) t += s_w[w];
  return t;
}

__global__ __launch_bounds__(kBaseThreads) void k_base_sums(int32_t n, const uint32_t* __restrict__ tiles_touched,
                                                            unsigned long long* __restrict__ bsum) {
  __shared__ unsigned long long s_w[kBaseThreads / 64];
  unsigned long long v = 0;
#pragma unroll
  for (int i = 0; i < kBaseItems; ++i) {
    const int64_t idx = (int64_t)blockIdx.x * kBaseTile + i * kBaseThreads + threadIdx.x;
    if (idx < n) v += tiles_touched[idx];
  }
  const unsigned long long t = block_sum_u64(v, s_w);
  if (threadIdx.x == 0) bsum[blockIdx.x] = t;
}

template <bool FROM_COUNTS>
__global__ __launch_bounds__(kBaseThreads) void k_base_scan(int32_t n, const uint32_t* __restrict__ tiles_touched,
                                                            const unsigned long long* __restrict__ bsum,
                                                            uint32_t* __restrict__ base,
                                                            unsigned long long* __restrict__ total) {
  __shared__ unsigned long long s_w[kBaseThreads / 64];
  __shared__ unsigned long long s_x[kBaseThreads / 64];
  // the totals of the blocks before this one: from k_base_sums, or (FROM_COUNTS) from the counts
  unsigned long long pre = 0;
  if (FROM_COUNTS) {
    const int64_t lim = (int64_t)blockIdx.x * kBaseTile;  // every id before the block (all < n)
    for (int64_t i = threadIdx.x; i < lim; i += 8 * kBaseThreads) {
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = i + k * kBaseThreads < lim ? tiles_touched[i + k * kBaseThreads] : 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) pre += v[k];
    }
  } else {
    for (uint32_t b = threadIdx.x; b < blockIdx.x; b += kBaseThreads) pre += bsum[b];
  }
  pre = block_sum_u64(pre, s_w);
  // exclusive scan of this block's 4096 counts, four consecutive ids per thread
  const int64_t i0 = (int64_t)blockIdx.x * kBaseTile + (int64_t)threadIdx.x * kBaseItems;
  uint32_t c[kBaseItems];
  unsigned long long own = 0;
#pragma unroll
  for (int i = 0; i < kBaseItems; ++i) {
    c[i] = i0 + i < n ? tiles_touched[i0 + i] : 0u;
    own += c[i];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long inc = own;
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long up = __shfl_up(inc, d);
    if (lane >= d) inc += up;
  }
  if (lane == 63) s_x[wave] = inc;
  __syncthreads();
  unsigned long long wpre = 0;
  for (int w = 0; w < wave; ++w) wpre += s_x[w];
  unsigned long long run = pre + wpre + inc - own;
#pragma unroll
  for (int i = 0; i < kBaseItems; ++i) {
    if (i0 + i < n) base[i0 + i] = (uint32_t)run;
    run += c[i];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == kBaseThreads - 1) *total = run;
}


}  // namespace
}  // namespace gs

using namespace gs;

namespace {
bool proj_ok(const gs_projected* p) {
  return p && p->d_means2d && p->d_conics && p->d_depths && p->d_opacities && p->d_colors && p->d_radii &&
         p->d_tiles_touched;
}
}  // namespace

extern "C" size_t gs_raster_workspace_bytes(void) {
  // per slot and pixel: (T, r, g, b), the depth channel's contribution, the chunk's transmittance
  // factor, its last added entry and stop flag; then the chunked forward's synchronisation words
  return (size_t)kPlanMaxSlots * kRasterThreads * (sizeof(float4) + 2 * sizeof(float) + sizeof(uint32_t)) +
         kRasterSyncWords * sizeof(uint32_t);
}

namespace {
gs_status rasterize_fwd(const char* name, int32_t n, const gs_projected* proj, const gs_camera* cam,
                        const uint32_t* d_ids, const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan,
                        void* d_raster_ws, float* d_image, float* d_depth, float* d_final_T, uint32_t* d_n_contrib,
                        const float* d_target, float* d_dL_dimage, uint64_t* d_eval_count, void* stream) {
  std::string why;
  const std::string nm = name;
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, nm + ": n < 0");
  if (!valid_camera(cam, &why)) return set_error(GS_ERR_INVALID_ARG, nm + ": " + why);
  if (!d_tile_ranges || !d_image || !d_final_T || !d_n_contrib)
    return set_error(GS_ERR_INVALID_ARG, nm + ": NULL output or ranges");
  if (n > 0 && (!proj_ok(proj) || !d_ids)) return set_error(GS_ERR_INVALID_ARG, nm + ": NULL input");
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  if (ntiles > ((int64_t)1 << 24)) return set_error(GS_ERR_LIMIT, nm + ": more than 2^24 tiles");
  const float l1_scale = 1.0f / (float)((size_t)cam->width * cam->height * 3);
  const DevCamera dc = to_dev(*cam);
  hipStream_t s = (hipStream_t)stream;
  {
    // with a plan and the raster workspace (a training forward) the checkpoints are stored and
    // tiles of three or more blended chunks (2 L entries) and more than 512 entries are blended
    // chunk by chunk in parallel
    const bool ck = d_raster_plan && d_raster_ws;
    const bool dep = d_depth != nullptr;
    auto pick = [&](auto c_, auto k_, auto d_) {
      return k_blend<decltype(c_)::value, decltype(k_)::value, decltype(d_)::value>;
    };
    using T1 = std::true_type;
    using F0 = std::false_type;
    auto kern = d_eval_count ? (ck ? (dep ? pick(T1{}, T1{}, T1{}) : pick(T1{}, T1{}, F0{}))
                                   : (dep ? pick(T1{}, F0{}, T1{}) : pick(T1{}, F0{}, F0{})))
                             : (ck ? (dep ? pick(F0{}, T1{}, T1{}) : pick(F0{}, T1{}, F0{}))
                                   : (dep ? pick(F0{}, F0{}, T1{}) : pick(F0{}, F0{}, F0{})));
    const RasterWs wsp = raster_ws_parts(ck ? d_raster_ws : nullptr);
    const float* m2 = n > 0 ? proj->d_means2d : nullptr;
    const float* co = n > 0 ? proj->d_conics : nullptr;
    const float* op = n > 0 ? proj->d_opacities : nullptr;
    const float* cl = n > 0 ? proj->d_colors : nullptr;
    const float* dp = n > 0 ? proj->d_depths : nullptr;
    {
      TimedScope ts("blend", s);
      // a training forward adds the split chunks (at most kPlanMaxSplit; the plan says how many)
      const unsigned grid = (unsigned)(ck ? ntiles + kPlanMaxSplit : ntiles);
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kRasterThreads), 0, s, (uint32_t)n, d_tile_ranges, d_raster_plan,
                         (uint32_t)ntiles, wsp, d_ids, m2, co, op, cl, dp, dc, d_image, d_depth, d_final_T,
                         d_n_contrib, (unsigned long long*)d_eval_count, d_target, d_dL_dimage, l1_scale);
    }
  }
  return check_launch(name);
}
}  // namespace

extern "C" gs_status gs_rasterize_fwd(int32_t n, const gs_projected* proj, const gs_camera* cam,
                                      const uint32_t* d_ids, const uint32_t* d_tile_ranges,
                                      const uint32_t* d_raster_plan, void* d_raster_ws, float* d_image,
                                      float* d_depth, float* d_final_T, uint32_t* d_n_contrib,
                                      uint64_t* d_eval_count, void* stream) {
  return rasterize_fwd("gs_rasterize_fwd", n, proj, cam, d_ids, d_tile_ranges, d_raster_plan, d_raster_ws, d_image,
                       d_depth, d_final_T, d_n_contrib, nullptr, nullptr, d_eval_count, stream);
}

extern "C" gs_status gs_rasterize_fwd_l1(int32_t n, const gs_projected* proj, const gs_camera* cam,
                                         const uint32_t* d_ids, const uint32_t* d_tile_ranges,
                                         const uint32_t* d_raster_plan, void* d_raster_ws, float* d_image,
                                         float* d_depth, float* d_final_T, uint32_t* d_n_contrib,
                                         const float* d_target, float* d_dL_dimage, uint64_t* d_eval_count,
                                         void* stream) {
  if (!d_target || !d_dL_dimage) return set_error(GS_ERR_INVALID_ARG, "gs_rasterize_fwd_l1: NULL target or gradient");
  return rasterize_fwd("gs_rasterize_fwd_l1", n, proj, cam, d_ids, d_tile_ranges, d_raster_plan, d_raster_ws,
                       d_image, d_depth, d_final_T, d_n_contrib, d_target, d_dL_dimage, d_eval_count, stream);
}

namespace {
// Workspace of the record modes: g2d [10, n] | base [n] u32 | total u64 | block sums u64 | rec [cap, 10]
struct BwdRecLayout {
  size_t g2d, base, total, bsum, rec, bytes;
};
BwdRecLayout bwd_rec_layout(int32_t n, int64_t cap) {
  BwdRecLayout L{};
  const size_t nb = ((size_t)n + kBaseTile - 1) / kBaseTile;
  L.g2d = 0;
  L.base = align_up(L.g2d + (size_t)n * kG2d * 4, 256);
  L.total = align_up(L.base + (size_t)n * 4, 256);
  L.bsum = align_up(L.total + 8, 256);
  L.rec = align_up(L.bsum + nb * 8, 256);
  L.bytes = align_up(L.rec + (size_t)cap * kG2d * 4 + 16, 256);
  return L;
}

gs_status rasterize_bwd(const char* name, int mode, int32_t n, int32_t sh_degree, const float* d_means,
                        const float* d_log_scales, const float* d_quats, const float* d_opacity_logits,
                        const float* d_sh, const gs_camera* cam, const gs_projected* proj, const uint32_t* d_ids,
                        const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan, const void* d_raster_ws,
                        const float* d_final_T, const uint32_t* d_n_contrib, const float* d_dL_dimage,
                        const float* d_dL_ddepth, int64_t pair_capacity, void* d_workspace, size_t workspace_bytes,
                        float* d_grad_means,
                        float* d_grad_log_scales, float* d_grad_quats, float* d_grad_opacity_logits,
                        float* d_grad_sh, float* d_grad_means2d, uint64_t* d_eval_count, void* stream) {
  const std::string nm = name;
  std::string why;
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, nm + ": n < 0");
  if (sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return set_error(GS_ERR_INVALID_ARG, nm + ": sh_degree not in 0..3");
  if (!valid_camera(cam, &why)) return set_error(GS_ERR_INVALID_ARG, nm + ": " + why);
  if (mode != kBwdAtomic && (pair_capacity < 0 || pair_capacity >= ((int64_t)1 << 30)))
    return set_error(pair_capacity < 0 ? GS_ERR_INVALID_ARG : GS_ERR_LIMIT, nm + ": pair_capacity not in [0, 2^30)");
  if (n == 0) return GS_OK;
  if (!d_means || !d_log_scales || !d_quats || !d_opacity_logits || !d_sh || !proj_ok(proj) || !d_ids ||
      !d_tile_ranges || !d_final_T || !d_n_contrib || !d_dL_dimage || !d_grad_means || !d_grad_log_scales ||
      !d_grad_quats || !d_grad_opacity_logits || !d_grad_sh)
    return set_error(GS_ERR_INVALID_ARG, nm + ": NULL pointer with n > 0");
  const BwdRecLayout RL = bwd_rec_layout(n, pair_capacity);
  const size_t need = mode == kBwdAtomic ? gs_bwd_workspace_bytes(n) : RL.bytes;
  if (!d_workspace || workspace_bytes < need)
    return set_error(GS_ERR_INVALID_ARG, nm + ": workspace smaller than its size function");
  if (mode != kBwdAtomic && (reinterpret_cast<uintptr_t>(d_workspace) & 255) != 0)
    return set_error(GS_ERR_INVALID_ARG, nm + ": workspace must be 256-byte aligned");
  if (((reinterpret_cast<uintptr_t>(d_quats) | reinterpret_cast<uintptr_t>(d_grad_quats)) & 15) != 0)
    return set_error(GS_ERR_INVALID_ARG, nm + ": quaternion arrays must be 16-byte aligned");
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  if (ntiles > ((int64_t)1 << 24)) return set_error(GS_ERR_LIMIT, nm + ": more than 2^24 tiles");
  const DevCamera dc = to_dev(*cam);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)d_workspace;
  float* g2d = (float*)(ws + RL.g2d);
  uint32_t* base = nullptr;
  unsigned long long* total = nullptr;
  float* rec = nullptr;
  if (mode == kBwdAtomic) {
    TimedScope ts("bwd_zero", s);
    const size_t count = (size_t)n * kG2d;
    const unsigned blocks = (unsigned)((count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, s, g2d, count);
  } else {
    TimedScope ts("bwd_base", s);
    base = (uint32_t*)(ws + RL.base);
    total = (unsigned long long*)(ws + RL.total);
    rec = (float*)(ws + RL.rec);
    unsigned long long* bsum = (unsigned long long*)(ws + RL.bsum);
    const unsigned nb = (unsigned)(((size_t)n + kBaseTile - 1) / kBaseTile);
    if (nb <= kBaseOne) {
      hipLaunchKernelGGL(k_base_scan<true>, dim3(nb), dim3(kBaseThreads), 0, s, n, proj->d_tiles_touched, bsum, base,
                         total);
    } else {
      hipLaunchKernelGGL(k_base_sums, dim3(nb), dim3(kBaseThreads), 0, s, n, proj->d_tiles_touched, bsum);
      hipLaunchKernelGGL(k_base_scan<false>, dim3(nb), dim3(kBaseThreads), 0, s, n, proj->d_tiles_touched, bsum, base,
                         total);
    }
  }
  {
    TimedScope ts("rbwd", s);
    auto pick = [&](auto count_tag, auto depth_tag) {
      constexpr bool C = decltype(count_tag)::value, D = decltype(depth_tag)::value;
      return mode == kBwdAtomic ? k_rbwd<C, kBwdAtomic, D> : k_rbwd<C, kBwdDeterministic, D>;
    };
    const bool dep = d_dL_ddepth != nullptr;
    auto kern = d_eval_count ? (dep ? pick(std::true_type{}, std::true_type{}) : pick(std::true_type{}, std::false_type{}))
                             : (dep ? pick(std::false_type{}, std::true_type{}) : pick(std::false_type{}, std::false_type{}));
    // with checkpoints: one workgroup per work item of the plan (the extra ones, fewer than
    // kPlanMaxChunks, then one per tile)
    const bool chunked = d_raster_plan && d_raster_ws;
    const unsigned grid = (unsigned)(chunked ? ntiles + kPlanMaxChunks : ntiles);
    const float4* ws4 = chunked ? (const float4*)d_raster_ws : nullptr;
    const float* wsd = ws4 ? (const float*)(ws4 + (size_t)kPlanMaxSlots * kRasterThreads) : nullptr;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kRasterThreads), 0, s, (uint32_t)n, d_tile_ranges, d_raster_plan,
                       (uint32_t)ntiles, ws4, wsd, d_ids, proj->d_means2d, proj->d_conics, proj->d_opacities,
                       proj->d_colors, proj->d_depths, proj->d_radii, dc, d_final_T, d_n_contrib, d_dL_dimage,
                       d_dL_ddepth, g2d, base, rec, (uint32_t)pair_capacity, (unsigned long long*)d_eval_count);
  }
  {
    // with records (the deterministic backward) the chain rule's launch sums them first
    TimedScope ts("pbwd", s);
    const dim3 grid((n + 255) / 256), block(256);
    const bool seg = mode != kBwdAtomic;
#define GS_LAUNCH_PBWD(D)                                                                                        \
  hipLaunchKernelGGL((seg ? k_pbwd<D, true> : k_pbwd<D, false>), grid, block, 0, s, n, d_means, d_log_scales,     \
                     d_quats, d_opacity_logits, d_sh, dc, proj->d_tiles_touched, g2d, base, total, rec,          \
                     (uint32_t)pair_capacity, d_grad_means, d_grad_log_scales, d_grad_quats,                     \
                     d_grad_opacity_logits, d_grad_sh, d_grad_means2d)
    switch (sh_degree) {
      case 0: GS_LAUNCH_PBWD(0); break;
      case 1: GS_LAUNCH_PBWD(1); break;
      case 2: GS_LAUNCH_PBWD(2); break;
      default: GS_LAUNCH_PBWD(3); break;
    }
#undef GS_LAUNCH_PBWD
  }
  return check_launch(name);
}
}  // namespace

extern "C" size_t gs_bwd_workspace_bytes(int32_t n) {
  return n <= 0 ? 256 : align_up((size_t)n * kG2d * 4, 256);
}

extern "C" size_t gs_bwd_det_workspace_bytes(int32_t n, int64_t pair_capacity) {
  if (n < 0 || pair_capacity < 0 || pair_capacity >= ((int64_t)1 << 30)) return 0;
  return bwd_rec_layout(n, pair_capacity).bytes;
}

extern "C" gs_status gs_rasterize_bwd(int32_t n, int32_t sh_degree, const float* d_means,
                                      const float* d_log_scales, const float* d_quats,
                                      const float* d_opacity_logits, const float* d_sh, const gs_camera* cam,
                                      const gs_projected* proj, const uint32_t* d_ids,
                                      const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan,
                                      const void* d_raster_ws, const float* d_final_T,
                                      const uint32_t* d_n_contrib, const float* d_dL_dimage,
                                      const float* d_dL_ddepth, void* d_workspace, size_t workspace_bytes,
                                      float* d_grad_means, float* d_grad_log_scales, float* d_grad_quats,
                                      float* d_grad_opacity_logits, float* d_grad_sh, float* d_grad_means2d,
                                      uint64_t* d_eval_count, void* stream) {
  return rasterize_bwd("gs_rasterize_bwd", kBwdAtomic, n, sh_degree, d_means, d_log_scales, d_quats,
                       d_opacity_logits, d_sh, cam, proj, d_ids, d_tile_ranges, d_raster_plan, d_raster_ws, d_final_T,
                       d_n_contrib, d_dL_dimage, d_dL_ddepth, 0, d_workspace, workspace_bytes, d_grad_means,
                       d_grad_log_scales, d_grad_quats, d_grad_opacity_logits, d_grad_sh, d_grad_means2d,
                       d_eval_count, stream);
}

extern "C" gs_status gs_rasterize_bwd_deterministic(
    int32_t n, int32_t sh_degree, const float* d_means, const float* d_log_scales, const float* d_quats,
    const float* d_opacity_logits, const float* d_sh, const gs_camera* cam, const gs_projected* proj,
    const uint32_t* d_ids, const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan, const void* d_raster_ws,
    const float* d_final_T, const uint32_t* d_n_contrib, const float* d_dL_dimage, const float* d_dL_ddepth,
    int64_t pair_capacity, void* d_workspace, size_t workspace_bytes, float* d_grad_means, float* d_grad_log_scales,
    float* d_grad_quats, float* d_grad_opacity_logits, float* d_grad_sh, float* d_grad_means2d,
    uint64_t* d_eval_count, void* stream) {
  return rasterize_bwd("gs_rasterize_bwd_deterministic", kBwdDeterministic, n, sh_degree, d_means, d_log_scales,
                       d_quats, d_opacity_logits, d_sh, cam, proj, d_ids, d_tile_ranges, d_raster_plan, d_raster_ws,
                       d_final_T, d_n_contrib, d_dL_dimage, d_dL_ddepth, pair_capacity, d_workspace, workspace_bytes,
                       d_grad_means, d_grad_log_scales, d_grad_quats, d_grad_opacity_logits, d_grad_sh,
                       d_grad_means2d, d_eval_count, stream);
}

