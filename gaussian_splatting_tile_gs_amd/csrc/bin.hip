// Binning: count, emit, sort and range of tile/Gaussian pairs.
//
// What is computed ("SplatRs: The Week the Gap Closed", section "Throughput: the tile
// rasterizer": project, count, emit, sort, range): for every drawn Gaussian i and every tile of
// its rectangle, the pair (key = tile << 32 | float_bits(depth_i), value = i), the pairs sorted
// by key with equal keys in ascending i, and the per-tile [start, end) ranges.
//
// How (MI355X design, not the pages'): a full 64-bit key sort would take 6 radix passes over the
// pairs. Here the depth part is settled once per Gaussian instead of once per pair:
//   1. k_depth_prep     depth keys (culled -> 0xFFFFFFFF) + all four 8-bit digit histograms
//   2. 4 x k_onesweep   stable LSD radix sort of the N Gaussians by depth bits
//   3. k_scan           single-pass prefix scan of the tile counts in depth order -> offsets, P
//      (P is read back: the one host wait, also the capacity check)
//   4. k_emit           (tile id, i) pairs in depth order + the tile-digit histograms
//   5. ceil(bits/8) x k_onesweep  stable LSD radix sort of the pairs by tile id only; the last
//      pass writes the 64-bit key (tile << 32 | depth bits of i) and the id
//   6. k_ranges         per-tile [start, end)
// Emitting in (depth, id) order and sorting stably by tile gives exactly the (tile, depth, id)
// order of the stable 64-bit key sort, with 1-2 passes over the pairs instead of 6.
//
// Each radix pass is Onesweep-style (Adinets & Merrill, "Onesweep: A Faster Least Significant
// Digit Radix Sort for GPUs", 2022): digit histograms are known before the pass, and one kernel
// ranks a 4096-key tile in registers/LDS, publishes per-digit counts and resolves its global
// offsets by decoupled look-back over earlier tiles. Tiles take their index from an atomic
// ticket, so a tile only ever waits on tiles that have already started (no forward-progress
// assumption between workgroups). Ranking is stable: within a wave, equal digits are matched
// with eight 64-lane ballots; waves own contiguous 1024-key segments in index order.
//
// Bytes per pair (algorithmic): emit writes 8; each pair pass reads 8 and writes 8 (the last
// writes 12 and gathers 4); ranges read 8. With 2 pair passes that is 8 + 16 + 24 + 8 = 56 B/pair,
// plus ~40 B per Gaussian for the depth sort and scan.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;  // 4096 keys per workgroup
constexpr int kRadix = 256;
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagPre = 2ull << 62;
constexpr uint64_t kValMask = (1ull << 62) - 1;

// ---- control block at the start of the workspace ----
struct Ctrl {
  uint64_t num_pairs;
  uint32_t counters[16];        // tile tickets: [0..3] depth passes, [4..6] pair passes, [7] scan
  uint32_t hist_depth[4][kRadix];
  uint32_t hist_pair[3][kRadix];
};

__device__ __forceinline__ uint64_t ld_acquire_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan across a wave64 (Kogge-Stone over lane shuffles).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive scan of one value per thread over a 256-thread workgroup; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan256(uint32_t v, uint32_t* s_wsum, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
    const uint32_t x = s_wsum[w];
    before += (w < wave) ? x : 0u;
    sum += x;
  }
  __syncthreads();
  *total = sum;
  return before + inc - v;
}

// ---------------------------------------------------------------------------------------------
// 1. depth keys and the four digit histograms of the depth sort
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void k_depth_prep(int32_t n, const float* __restrict__ depths,
                                                             const uint32_t* __restrict__ tiles,
                                                             uint32_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                             Ctrl* ctrl) {
  __shared__ uint32_t s_hist[4][kRadix];
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) s_hist[p][tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kSortTile;
#pragma unroll 4
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = base + i * kSortThreads + tid;
    if (idx < n) {
      const uint32_t k = tiles[idx] > 0 ? __float_as_uint(depths[idx]) : 0xFFFFFFFFu;
      keys[idx] = k;
      vals[idx] = (uint32_t)idx;
#pragma unroll
      for (int p = 0; p < 4; ++p) atomicAdd(&s_hist[p][(k >> (8 * p)) & 0xFF], 1u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t c = s_hist[p][tid];
    if (c) atomicAdd(&ctrl->hist_depth[p][tid], c);
  }
}

// ---------------------------------------------------------------------------------------------
// 2/5. one stable LSD radix pass over `bits` (<= 8) bits at `shift` (Onesweep-style)
// ---------------------------------------------------------------------------------------------
template <bool FINAL>
__global__ __launch_bounds__(kSortThreads) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, uint64_t* __restrict__ out_keys64, const uint32_t* __restrict__ depth_bits,
    uint32_t n, int shift, int bits, const uint32_t* __restrict__ hist, uint64_t* __restrict__ status,
    uint32_t* __restrict__ ticket) {
  __shared__ uint32_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  __shared__ uint32_t s_wcnt[kSortWaves][kRadix];
  __shared__ uint32_t s_dpre[kRadix];
  __shared__ uint32_t s_goff[kRadix];
  __shared__ uint32_t s_wsum[kSortWaves];
  __shared__ uint32_t s_vb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_vb = atomicAdd(ticket, 1u);
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) s_wcnt[w][tid] = 0;
  __syncthreads();
  const uint32_t vb = s_vb;
  const uint32_t base = vb * (uint32_t)kSortTile;
  if (base >= n) return;  // only with a stale ticket counter; every launched tile has base < n
  const uint32_t mask = (1u << bits) - 1u;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- load (wave-striped: wave w owns [base + 1024 w, base + 1024 (w + 1))) and rank ----
  uint32_t k[kSortItems], v[kSortItems], rank[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    const bool valid = idx < n;
    k[i] = valid ? keys_in[idx] : 0u;
    v[i] = valid ? vals_in[idx] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    const bool valid = idx < n;
    const uint32_t d = (k[i] >> shift) & mask;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const uint32_t r = (uint32_t)__popcll(m & lt_mask);
    uint32_t pre = 0;
    if (valid) pre = s_wcnt[wave][d];
    rank[i] = pre + r;
    if (valid && r == 0) s_wcnt[wave][d] = pre + (uint32_t)__popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // ---- per digit: wave offsets, tile total, publish, look back ----
  const uint32_t c0 = s_wcnt[0][tid], c1 = s_wcnt[1][tid], c2 = s_wcnt[2][tid], c3 = s_wcnt[3][tid];
  const uint32_t tot = c0 + c1 + c2 + c3;
  uint64_t* my_status = status + (size_t)vb * kRadix + tid;
  st_release_dev(my_status, (vb == 0 ? kFlagPre : kFlagAgg) | (uint64_t)tot);
  uint32_t dummy;
  const uint32_t bucket_excl = block_excl_scan256(hist[tid], s_wsum, &dummy);
  const uint32_t dpre = block_excl_scan256(tot, s_wsum, &dummy);
  s_wcnt[0][tid] = 0;
  s_wcnt[1][tid] = c0;
  s_wcnt[2][tid] = c0 + c1;
  s_wcnt[3][tid] = c0 + c1 + c2;
  s_dpre[tid] = dpre;
  uint64_t excl = 0;
  if (vb > 0) {
    int64_t j = (int64_t)vb - 1;
    while (true) {
      const uint64_t st = ld_acquire_dev(status + (size_t)j * kRadix + tid);
      if ((st & ~kValMask) == 0) {
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      excl += st & kValMask;
      if ((st & ~kValMask) == kFlagPre) break;
      --j;
    }
    st_release_dev(my_status, kFlagPre | (excl + tot));
  }
  s_goff[tid] = bucket_excl + (uint32_t)excl - dpre;
  __syncthreads();

  // ---- scatter to LDS in local sorted order, then out with consecutive threads ----
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    if (idx < n) {
      const uint32_t d = (k[i] >> shift) & mask;
      const uint32_t lp = s_dpre[d] + s_wcnt[wave][d] + rank[i];
      s_keys[lp] = k[i];
      s_vals[lp] = v[i];
    }
  }
  __syncthreads();
  const uint32_t count = (n - base < (uint32_t)kSortTile) ? (n - base) : (uint32_t)kSortTile;
  for (uint32_t j = tid; j < count; j += kSortThreads) {
    const uint32_t key = s_keys[j], val = s_vals[j];
    const uint32_t gp = s_goff[(key >> shift) & mask] + j;
    if (gp >= n) continue;  // cannot happen when the histogram matches the keys; never write past n
    if (FINAL) {
      out_keys64[gp] = ((uint64_t)key << 32) | (uint64_t)depth_bits[val];
      vals_out[gp] = val;
    } else {
      keys_out[gp] = key;
      vals_out[gp] = val;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 3. exclusive scan of tiles_touched in depth order (single pass, decoupled look-back)
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void k_scan(int32_t n, const uint32_t* __restrict__ sorted_ids,
                                                       const uint32_t* __restrict__ tiles,
                                                       uint32_t* __restrict__ offsets, uint64_t* __restrict__ status,
                                                       Ctrl* ctrl) {
  __shared__ uint32_t s_wsum[kSortWaves];
  __shared__ uint32_t s_vb;
  __shared__ uint64_t s_excl;
  const int tid = threadIdx.x;
  if (tid == 0) s_vb = atomicAdd(&ctrl->counters[7], 1u);
  __syncthreads();
  const uint32_t vb = s_vb;
  const int base = (int)vb * kSortTile + tid * kSortItems;  // blocked: 16 consecutive per thread
  uint32_t c[kSortItems];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = base + i;
    c[i] = idx < n ? tiles[sorted_ids[idx]] : 0u;
    sum += c[i];
  }
  uint32_t tot;
  const uint32_t texcl = block_excl_scan256(sum, s_wsum, &tot);
  if (tid == 0) {
    uint64_t excl = 0;
    st_release_dev(status + vb, (vb == 0 ? kFlagPre : kFlagAgg) | (uint64_t)tot);
    if (vb > 0) {
      int64_t j = (int64_t)vb - 1;
      while (true) {
        const uint64_t st = ld_acquire_dev(status + j);
        if ((st & ~kValMask) == 0) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        excl += st & kValMask;
        if ((st & ~kValMask) == kFlagPre) break;
        --j;
      }
      st_release_dev(status + vb, kFlagPre | (excl + tot));
    }
    s_excl = excl;
    if ((uint64_t)(vb + 1) * kSortTile >= (uint64_t)n) ctrl->num_pairs = excl + tot;  // last tile
  }
  __syncthreads();
  uint64_t run = s_excl + texcl;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = base + i;
    if (idx < n) offsets[idx] = (uint32_t)run;
    run += c[i];
  }
}

// ---------------------------------------------------------------------------------------------
// 4. emit (tile id, Gaussian id) pairs in depth order, with the tile-digit histograms
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(int32_t n, const uint32_t* __restrict__ sorted_ids,
                                              const uint32_t* __restrict__ offsets, const uint32_t* __restrict__ tiles,
                                              const float* __restrict__ means2d, const int32_t* __restrict__ radii,
                                              int32_t tiles_x, int32_t tiles_y, uint32_t* __restrict__ pkeys,
                                              uint32_t* __restrict__ pvals, uint32_t num_pairs, int npass,
                                              Ctrl* ctrl) {
  __shared__ uint32_t s_hist[3][kRadix];
  const int tid = threadIdx.x;
  for (int p = 0; p < npass; ++p) s_hist[p][tid] = 0;
  __syncthreads();
  const int i = blockIdx.x * 256 + tid;
  if (i < n) {
    const uint32_t g = sorted_ids[i];
    const uint32_t cnt = tiles[g];
    if (cnt > 0) {
      const float2 m = *reinterpret_cast<const float2*>(means2d + 2 * g);
      const int2 r = *reinterpret_cast<const int2*>(radii + 2 * g);
      const TileRect rc = tile_rect(m.x, m.y, (float)r.x, (float)r.y, tiles_x, tiles_y);
      uint32_t o = offsets[i];
      const uint32_t end = (o + cnt < num_pairs) ? o + cnt : num_pairs;
      for (int ty = rc.y0; ty < rc.y1 && o < end; ++ty)
        for (int tx = rc.x0; tx < rc.x1 && o < end; ++tx, ++o) {
          const uint32_t t = (uint32_t)(ty * tiles_x + tx);
          pkeys[o] = t;
          pvals[o] = g;
          for (int p = 0; p < npass; ++p) atomicAdd(&s_hist[p][(t >> (8 * p)) & 0xFF], 1u);
        }
    }
  }
  __syncthreads();
  for (int p = 0; p < npass; ++p) {
    const uint32_t c = s_hist[p][tid];
    if (c) atomicAdd(&ctrl->hist_pair[p][tid], c);
  }
}

// ---------------------------------------------------------------------------------------------
// 6. per-tile ranges from the sorted 64-bit keys (ranges zeroed beforehand)
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ranges(uint32_t P, const uint64_t* __restrict__ keys, uint32_t ntiles,
                                                uint32_t* __restrict__ ranges) {
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;
  if (i >= P) return;
  const uint32_t t = (uint32_t)(keys[i] >> 32);
  if (t >= ntiles) return;
  if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * t] = i;
  if (i == P - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * t + 1] = i + 1;
}

// ---------------------------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------------------------
struct BinLayout {
  size_t ctrl, dkA, dvA, dkB, dvB, offsets, scan_status, dstatus, pkB, pvB, pstatus, total;
  uint32_t nbN, nbCap;
  int tile_bits, npass;
};

BinLayout bin_layout(int32_t n, int64_t cap, const gs_camera* cam) {
  BinLayout L{};
  const size_t A = 256;
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  int tb = 1;
  while (((int64_t)1 << tb) < ntiles) ++tb;
  L.tile_bits = tb;
  L.npass = (tb + 7) / 8;
  L.nbN = (uint32_t)((n + kSortTile - 1) / kSortTile);
  L.nbCap = (uint32_t)((cap + kSortTile - 1) / kSortTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, A);
    return at;
  };
  // the control block and the depth/scan look-back words come first: one memset clears them
  L.ctrl = take(sizeof(Ctrl));
  L.scan_status = take((size_t)L.nbN * 8);
  L.dstatus = take((size_t)4 * L.nbN * kRadix * 8);
  L.dkA = take((size_t)n * 4);
  L.dvA = take((size_t)n * 4);
  L.dkB = take((size_t)n * 4);
  L.dvB = take((size_t)n * 4);
  L.offsets = take((size_t)n * 4);
  L.pkB = take((size_t)cap * 4);
  L.pvB = take((size_t)cap * 4);
  L.pstatus = take((size_t)L.npass * L.nbCap * kRadix * 8);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_bin_workspace_bytes(int32_t n, int64_t pair_capacity, const gs_camera* cam) {
  if (n < 0 || pair_capacity < 0 || !cam || cam->width <= 0 || cam->height <= 0) return 0;
  return bin_layout(n, pair_capacity, cam).total;
}

extern "C" gs_status gs_bin_and_sort(int32_t n, const gs_projected* proj, const gs_camera* cam, void* d_workspace,
                                     size_t workspace_bytes, int64_t pair_capacity, uint64_t* d_keys,
                                     uint32_t* d_ids, uint32_t* d_tile_ranges, int64_t* h_num_pairs, void* stream) {
  std::string why;
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: n < 0");
  if (!valid_camera(cam, &why)) return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: " + why);
  if (!h_num_pairs || !d_tile_ranges || pair_capacity < 0)
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL h_num_pairs/d_tile_ranges or capacity < 0");
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  if (ntiles > ((int64_t)1 << 24)) return set_error(GS_ERR_LIMIT, "gs_bin_and_sort: more than 2^24 tiles");
  if (pair_capacity > 0 && (!d_keys || !d_ids))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL d_keys/d_ids with capacity > 0");
  if (n > 0 && (!proj || !proj->d_depths || !proj->d_tiles_touched || !proj->d_means2d || !proj->d_radii))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL projected record with n > 0");
  const BinLayout L = bin_layout(n, pair_capacity, cam);
  if (n > 0 && (!d_workspace || workspace_bytes < L.total))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: workspace smaller than gs_bin_workspace_bytes()");
  if (((reinterpret_cast<uintptr_t>(d_workspace) & 255) != 0) || ((reinterpret_cast<uintptr_t>(d_keys) & 7) != 0))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: workspace must be 256-byte aligned, d_keys 8-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)d_workspace;
  *h_num_pairs = 0;
  if (n == 0) {
    if (hipMemsetAsync(d_tile_ranges, 0, (size_t)ntiles * 8, s) != hipSuccess) return check_launch("gs_bin_and_sort");
    return check_launch("gs_bin_and_sort");
  }
  Ctrl* ctrl = (Ctrl*)(ws + L.ctrl);
  uint32_t *dkA = (uint32_t*)(ws + L.dkA), *dvA = (uint32_t*)(ws + L.dvA), *dkB = (uint32_t*)(ws + L.dkB),
           *dvB = (uint32_t*)(ws + L.dvB), *offsets = (uint32_t*)(ws + L.offsets);
  uint64_t* scan_status = (uint64_t*)(ws + L.scan_status);
  uint64_t* dstatus = (uint64_t*)(ws + L.dstatus);
  // control block, depth-sort and scan look-back words start at zero
  if (hipMemsetAsync(ws, 0, L.dstatus + (size_t)4 * L.nbN * kRadix * 8 - L.ctrl, s) != hipSuccess)
    return check_launch("gs_bin_and_sort: memset");
  {
    TimedScope ts("depth_prep", s);
    hipLaunchKernelGGL(k_depth_prep, dim3(L.nbN), dim3(kSortThreads), 0, s, n, proj->d_depths,
                       proj->d_tiles_touched, dkA, dvA, ctrl);
  }
  for (int p = 0; p < 4; ++p) {
    const bool even = (p % 2) == 0;
    TimedScope ts("depth_sort_pass", s);
    hipLaunchKernelGGL(k_onesweep<false>, dim3(L.nbN), dim3(kSortThreads), 0, s, even ? dkA : dkB, even ? dvA : dvB,
                       even ? dkB : dkA, even ? dvB : dvA, (uint64_t*)nullptr, (const uint32_t*)nullptr,
                       (uint32_t)n, 8 * p, 8, ctrl->hist_depth[p], dstatus + (size_t)p * L.nbN * kRadix,
                       &ctrl->counters[p]);
  }
  {
    TimedScope ts("scan", s);
    hipLaunchKernelGGL(k_scan, dim3(L.nbN), dim3(kSortThreads), 0, s, n, dvA, proj->d_tiles_touched, offsets,
                       scan_status, ctrl);
  }
  uint64_t P = 0;
  if (hipMemcpyAsync(&P, &ctrl->num_pairs, sizeof(P), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return check_launch("gs_bin_and_sort: reading the pair count");
  *h_num_pairs = (int64_t)P;
  if ((int64_t)P > pair_capacity) {
    return set_error(GS_ERR_CAPACITY, "gs_bin_and_sort: " + std::to_string(P) + " pairs exceed the capacity " +
                                          std::to_string(pair_capacity));
  }
  if (P >= (1ull << 31)) return set_error(GS_ERR_LIMIT, "gs_bin_and_sort: 2^31 or more pairs");
  if (hipMemsetAsync(d_tile_ranges, 0, (size_t)ntiles * 8, s) != hipSuccess) return check_launch("gs_bin_and_sort");
  if (P == 0) return check_launch("gs_bin_and_sort");

  const uint32_t nbP = (uint32_t)((P + kSortTile - 1) / kSortTile);
  uint64_t* pstatus = (uint64_t*)(ws + L.pstatus);
  for (int p = 0; p < L.npass; ++p)
    if (hipMemsetAsync(pstatus + (size_t)p * L.nbCap * kRadix, 0, (size_t)nbP * kRadix * 8, s) != hipSuccess)
      return check_launch("gs_bin_and_sort: memset");
  // ping-pong: A = d_keys viewed as two u32 arrays of pair_capacity, B = workspace
  uint32_t* kA = (uint32_t*)d_keys;
  uint32_t* vA = kA + pair_capacity;
  uint32_t *kB = (uint32_t*)(ws + L.pkB), *vB = (uint32_t*)(ws + L.pvB);
  const bool emit_to_A = (L.npass % 2) == 0;
  const int32_t tiles_x = (cam->width + 15) / 16, tiles_y = (cam->height + 15) / 16;
  {
    TimedScope ts("emit", s);
    hipLaunchKernelGGL(k_emit, dim3((n + 255) / 256), dim3(256), 0, s, n, dvA, offsets, proj->d_tiles_touched,
                       proj->d_means2d, proj->d_radii, tiles_x, tiles_y, emit_to_A ? kA : kB,
                       emit_to_A ? vA : vB, (uint32_t)P, L.npass, ctrl);
  }
  bool in_A = emit_to_A;
  for (int p = 0; p < L.npass; ++p) {
    const int shift = 8 * p;
    const int bits = (L.tile_bits - shift) < 8 ? (L.tile_bits - shift) : 8;
    const bool last = p == L.npass - 1;
    uint32_t *ki = in_A ? kA : kB, *vi = in_A ? vA : vB;
    uint32_t *ko = in_A ? kB : kA, *vo = in_A ? vB : vA;
    TimedScope ts("pair_sort_pass", s);
    if (last) {
      hipLaunchKernelGGL(k_onesweep<true>, dim3(nbP), dim3(kSortThreads), 0, s, ki, vi, (uint32_t*)nullptr, d_ids,
                         d_keys, (const uint32_t*)proj->d_depths, (uint32_t)P, shift, bits, ctrl->hist_pair[p],
                         pstatus + (size_t)p * L.nbCap * kRadix, &ctrl->counters[4 + p]);
    } else {
      hipLaunchKernelGGL(k_onesweep<false>, dim3(nbP), dim3(kSortThreads), 0, s, ki, vi, ko, vo,
                         (uint64_t*)nullptr, (const uint32_t*)nullptr, (uint32_t)P, shift, bits, ctrl->hist_pair[p],
                         pstatus + (size_t)p * L.nbCap * kRadix, &ctrl->counters[4 + p]);
    }
    in_A = !in_A;
  }
  {
    TimedScope ts("ranges", s);
    hipLaunchKernelGGL(k_ranges, dim3((uint32_t)((P + 255) / 256)), dim3(256), 0, s, (uint32_t)P, d_keys,
                       (uint32_t)ntiles, d_tile_ranges);
  }
  return check_launch("gs_bin_and_sort");
}
