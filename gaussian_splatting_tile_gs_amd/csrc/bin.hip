// Binning: count, emit, sort and range of tile/Gaussian pairs.
//
// What is computed ("SplatRs: The Week the Gap Closed", section "Throughput: the tile
// rasterizer": project, count, emit, sort, range): for every drawn Gaussian i and every tile of
// its rectangle, the pair (key = tile << 32 | float_bits(depth_i), value = i), the pairs sorted
// by key with equal keys in ascending i, and the per-tile [start, end) ranges.
//
// How (MI355X design, not the pages'): a full 64-bit key sort would take 6 radix passes over the
// pairs. Here the depth part is settled once per Gaussian instead of once per pair:
//   1. k_bin_prep     depth keys (culled -> 0xFFFFFFFF), per-workgroup digit histograms of the
//                     four depth passes, and the zeroing of every counter, look-back word and
//                     tile range the later kernels rely on (no memset nodes, no host wait)
//   2. k_hist_reduce  the per-workgroup depth histograms summed (beyond 32 workgroups; below
//                     that each depth pass sums them itself)
//   3. 4 x k_onesweep stable LSD radix sort of the N Gaussians by depth bits
//   4. k_scan_emit    single-pass prefix scan of the tile counts in depth order; each workgroup
//                     then writes its Gaussians' (tile id, i) pairs with all 256 lanes sharing
//                     the work (coalesced, balanced however uneven the counts), accumulates the
//                     tile-digit histograms, and the last workgroup publishes P
//   5. ceil(bits/8) x k_onesweep  stable LSD radix sort of the pairs by tile id only; the last
//                     pass writes the 64-bit key (tile << 32 | depth bits of i) and the id
//   6. k_ranges       per-tile [start, end)
// Emitting in (depth, id) order and sorting stably by tile gives exactly the (tile, depth, id)
// order of the stable 64-bit key sort, with 1-2 passes over the pairs instead of 6. P never has
// to reach the host: the pair kernels are sized by the capacity and their workgroups stop at the
// device-side count (0 when P exceeds the capacity, which leaves every range empty).
//
// Each radix pass is Onesweep-style (Adinets & Merrill, "Onesweep: A Faster Least Significant
// Digit Radix Sort for GPUs", 2022): digit histograms are known before the pass, and one kernel
// ranks a 4096-key tile in registers/LDS, publishes per-digit counts and resolves its global
// offsets by decoupled look-back over earlier tiles. Tiles take their index from an atomic
// ticket, so a tile only ever waits on tiles that have already started (no forward-progress
// assumption between workgroups). Ranking is stable: within a wave, equal digits are matched
// with eight 64-lane ballots; the 16 waves of a workgroup own contiguous 256-key segments in
// index order (four keys per lane keep each wave's ranking chain short).
//
// Bytes per pair (algorithmic): emit writes 8; each pair pass reads 8 and writes 8 (the last
// writes 12 and gathers 4); ranges read 8. With 2 pair passes that is 8 + 16 + 24 + 8 = 56 B/pair,
// plus ~40 B per Gaussian for the depth sort and scan.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kSortThreads = 1024;  // 16 waves: short per-wave ranking chains
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 4;
constexpr int kSortTile = kSortThreads * kSortItems;  // 4096 keys per workgroup
constexpr int kScanTile = 256;                        // Gaussians per scan/emit workgroup
constexpr int kRadix = 256;
// Radix-pass look-back words are 32 bits: [31:30] flag (0 not ready, 1 tile aggregate,
// 2 inclusive prefix), [29:0] count, so sorted sequences are limited to below 2^30 elements.
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagPre = 2u << 30;
constexpr uint32_t kValMask = (1u << 30) - 1u;
// The scan's look-back words are 64 bits with the flag in [63:62]: P itself may exceed 2^32.
constexpr uint64_t kFlagAgg64 = 1ull << 62;
constexpr uint64_t kFlagPre64 = 2ull << 62;
constexpr uint64_t kValMask64 = (1ull << 62) - 1;

struct Ctrl {
  uint64_t num_pairs;    // P
  uint64_t eff_pairs;    // P if it fits the capacity, else 0: what the pair kernels process
  uint32_t tickets[16];  // [0..3] depth passes, [4..6] pair passes, [7] scan
  uint32_t hist_depth[4][kRadix];
  uint32_t hist_pair[3][kRadix];
};

template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan across a wave64 (Kogge-Stone over lane shuffles).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive scan over the values of the first 256 threads of the workgroup (the others pass 0);
// *total gets the sum. Every thread of the workgroup calls it (it holds two barriers).
template <typename T>
__device__ __forceinline__ T block_excl_scan256(T v, T* s_wsum, T* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T inc = wave_incl_scan<T>(v, lane);
  if (wave < 4 && lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  T before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const T x = s_wsum[w];
    before += (w < wave) ? x : T(0);
    sum += x;
  }
  __syncthreads();
  *total = sum;
  return before + inc - v;
}

// Decoupled look-back: the inclusive prefix of the tiles before `vb` in one column of look-back
// words. W predecessor words are read at once (independent loads, one round trip) and consumed
// nearest first until an inclusive prefix is found; a word not yet published stops the
// consumption and the window is read again from there. Every earlier tile has taken its ticket
// before this one, so every wait ends; tile 0 always publishes an inclusive prefix.
template <int W, typename T, T kFlagMask, T kPre, T kVal>
__device__ __forceinline__ T look_back(const T* status, uint32_t vb, int stride) {
  T excl = 0;
  int64_t j = (int64_t)vb - 1;
  while (true) {
    T st[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int64_t p = j - i;
      st[i] = p >= 0 ? ld_dev(status + (size_t)p * stride) : kPre;  // below tile 0: never consumed
    }
    int i = 0;
    for (; i < W; ++i) {
      const T f = st[i] & kFlagMask;
      if (f == 0) break;
      excl += st[i] & kVal;
      if (f == kPre) return excl;
    }
    j -= i;
    if (i < W) __builtin_amdgcn_s_sleep(1);
  }
}

// ---------------------------------------------------------------------------------------------
// 1. depth keys, per-workgroup digit histograms of the depth passes, zeroing
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void k_bin_prep(int32_t n, const float* __restrict__ depths,
                                                           const uint32_t* __restrict__ tiles,
                                                           uint32_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                           uint32_t* __restrict__ dhist, uint32_t nbN,
                                                           uint32_t* __restrict__ zero_a, size_t zero_a_words,
                                                           uint32_t* __restrict__ zero_b, size_t zero_b_words) {
  __shared__ uint32_t s_hist[4][kRadix];
  const int tid = threadIdx.x;
  const size_t gsz = (size_t)gridDim.x * kSortThreads;
  for (size_t i = blockIdx.x * (size_t)kSortThreads + tid; i < zero_a_words; i += gsz) zero_a[i] = 0u;
  for (size_t i = blockIdx.x * (size_t)kSortThreads + tid; i < zero_b_words; i += gsz) zero_b[i] = 0u;
  if (blockIdx.x >= nbN) return;  // workgroup-uniform
  if (tid < kRadix) {
#pragma unroll
    for (int p = 0; p < 4; ++p) s_hist[p][tid] = 0;
  }
  __syncthreads();
  const int base = blockIdx.x * kSortTile;
  uint32_t k[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {  // all loads in flight before any is used
    const int idx = base + i * kSortThreads + tid;
    const uint32_t t = idx < n ? tiles[idx] : 0u;
    const float z = idx < n ? depths[idx] : 0.0f;
    k[i] = t > 0 ? __float_as_uint(z) : 0xFFFFFFFFu;
  }
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = base + i * kSortThreads + tid;
    if (idx < n) {
      keys[idx] = k[i];
      vals[idx] = (uint32_t)idx;
#pragma unroll
      for (int p = 0; p < 4; ++p) atomicAdd(&s_hist[p][(k[i] >> (8 * p)) & 0xFF], 1u);
    }
  }
  __syncthreads();
  if (tid < kRadix) {
#pragma unroll
    for (int p = 0; p < 4; ++p) dhist[((size_t)blockIdx.x * 4 + p) * kRadix + tid] = s_hist[p][tid];
  }
}

// ---------------------------------------------------------------------------------------------
// 2. sum of the per-workgroup depth histograms: blockIdx.x = pass, blockIdx.y = chunk of rows
// (ctrl->hist_depth was zeroed by k_bin_prep)
// ---------------------------------------------------------------------------------------------
constexpr int kReduceRows = 64;
constexpr int kDirectHistRows = 32;
__global__ __launch_bounds__(kRadix) void k_hist_reduce(const uint32_t* __restrict__ dhist, uint32_t nbN, Ctrl* ctrl) {
  const int p = blockIdx.x, d = threadIdx.x;
  const uint32_t r0 = blockIdx.y * kReduceRows;
  const uint32_t r1 = (r0 + kReduceRows < nbN) ? r0 + kReduceRows : nbN;
  uint32_t s = 0;
  for (uint32_t r = r0; r < r1; ++r) s += dhist[((size_t)r * 4 + p) * kRadix + d];
  if (s) atomicAdd(&ctrl->hist_depth[p][d], s);
}

// ---------------------------------------------------------------------------------------------
// 3/5. one stable LSD radix pass over `bits` (<= 8) bits at `shift` (Onesweep-style)
// The element count is *n_dev when given (pairs: grid sized by the capacity), else n_host. The
// pass's digit histogram is the sum of `hist_parts` rows of 256 counts, `hist_stride` apart.
// ---------------------------------------------------------------------------------------------
template <bool FINAL>
__global__ __launch_bounds__(kSortThreads) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, uint64_t* __restrict__ out_keys64, const uint32_t* __restrict__ depth_bits,
    uint32_t n_host, const uint64_t* __restrict__ n_dev, int shift, int bits, const uint32_t* __restrict__ hist,
    int hist_parts, int hist_stride, uint32_t* __restrict__ status, uint32_t* __restrict__ ticket) {
  __shared__ uint32_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  __shared__ uint32_t s_wcnt[kSortWaves][kRadix];  // per wave and digit: count, then wave offset
  __shared__ uint32_t s_dpre[kRadix];
  __shared__ uint32_t s_goff[kRadix];
  __shared__ uint32_t s_wsum[4];
  __shared__ uint32_t s_vb;

  const uint32_t n = n_dev ? (uint32_t)*n_dev : n_host;
  if ((uint64_t)blockIdx.x * kSortTile >= n) return;  // workgroup-uniform: idle workgroups take no ticket
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_vb = atomicAdd(ticket, 1u);
  for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  // exactly ceil(n / 4096) workgroups take tickets, so every ticket has base < n
  const uint32_t vb = s_vb;
  const uint32_t base = vb * (uint32_t)kSortTile;
  if (base >= n) return;  // unreachable with a zeroed ticket; guards a stale one
  const uint32_t mask = (1u << bits) - 1u;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- load (wave-striped: wave w owns [base + 256 w, base + 256 (w + 1))) and rank ----
  uint32_t k[kSortItems], v[kSortItems], rank[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    const bool valid = idx < n;
    k[i] = valid ? keys_in[idx] : 0u;
    v[i] = valid ? vals_in[idx] : 0u;
  }
  uint32_t h = 0;  // the pass's histogram, read while the keys arrive
  if (tid < kRadix)
    for (int r = 0; r < hist_parts; ++r) h += hist[(size_t)r * hist_stride + tid];
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

  // ---- per digit (threads 0-255): wave offsets, tile total, publish, look back ----
  uint32_t tot = 0;
  if (tid < kRadix) {
    uint32_t c[kSortWaves];
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) c[w] = s_wcnt[w][tid];
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      s_wcnt[w][tid] = tot;
      tot += c[w];
    }
    st_dev(status + (size_t)vb * kRadix + tid, (vb == 0 ? kFlagPre : kFlagAgg) | tot);
  }
  uint32_t dummy;
  const uint32_t bucket_excl = block_excl_scan256<uint32_t>(h, s_wsum, &dummy);
  const uint32_t dpre = block_excl_scan256<uint32_t>(tot, s_wsum, &dummy);
  if (tid < kRadix) {
    s_dpre[tid] = dpre;
    uint32_t excl = 0;
    if (vb > 0) {
      excl = look_back<8, uint32_t, ~kValMask, kFlagPre, kValMask>(status + tid, vb, kRadix);
      st_dev(status + (size_t)vb * kRadix + tid, kFlagPre | (excl + tot));
    }
    s_goff[tid] = bucket_excl + excl - dpre;
  }
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
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t j = (uint32_t)(i * kSortThreads + tid);
    if (j >= count) break;
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
// 4. exclusive scan of tiles_touched in depth order (single pass, decoupled look-back) and
// emission of each workgroup's (tile id, Gaussian id) pairs, all 256 lanes sharing the pairs
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kScanTile) void k_scan_emit(
    int32_t n, const uint32_t* __restrict__ sorted_ids, const uint32_t* __restrict__ tiles,
    const float* __restrict__ means2d, const int32_t* __restrict__ radii, int32_t tiles_x, int32_t tiles_y,
    uint32_t* __restrict__ pkeys, uint32_t* __restrict__ pvals, uint64_t capacity, int npass,
    uint64_t* __restrict__ status, Ctrl* ctrl, int64_t* __restrict__ user_num_pairs) {
  __shared__ uint64_t s_wsum[4];
  __shared__ uint32_t s_incl[kScanTile];  // workgroup-inclusive pair counts, saturated at 2^31
  __shared__ uint32_t s_g[kScanTile];
  __shared__ int32_t s_x0[kScanTile], s_y0[kScanTile], s_w[kScanTile];
  __shared__ uint32_t s_hist[3][kRadix];
  __shared__ uint32_t s_vb;
  __shared__ uint64_t s_excl;
  const int tid = threadIdx.x;
  if (tid == 0) s_vb = atomicAdd(&ctrl->tickets[7], 1u);
  for (int p = 0; p < npass; ++p) s_hist[p][tid] = 0;
  __syncthreads();
  const uint32_t vb = s_vb;
  const int idx = (int)vb * kScanTile + tid;
  uint32_t g = 0, c = 0;
  if (idx < n) {
    g = sorted_ids[idx];
    c = tiles[g];
  }
  int32_t x0 = 0, y0 = 0, w = 1;
  if (c > 0) {
    const float2 m = *reinterpret_cast<const float2*>(means2d + 2 * g);
    const int2 r = *reinterpret_cast<const int2*>(radii + 2 * g);
    const TileRect rc = tile_rect(m.x, m.y, (float)r.x, (float)r.y, tiles_x, tiles_y);
    x0 = rc.x0;
    y0 = rc.y0;
    w = rc.x1 - rc.x0;
  }
  s_g[tid] = g;
  s_x0[tid] = x0;
  s_y0[tid] = y0;
  s_w[tid] = w;
  uint64_t tot;
  const uint64_t texcl = block_excl_scan256<uint64_t>((uint64_t)c, s_wsum, &tot);
  const uint64_t tincl = texcl + c;
  s_incl[tid] = tincl < 0x80000000ull ? (uint32_t)tincl : 0x80000000u;
  if (tid == 0) {
    st_dev(status + vb, (vb == 0 ? kFlagPre64 : kFlagAgg64) | tot);
    uint64_t excl = 0;
    if (vb > 0) {
      excl = look_back<16, uint64_t, ~kValMask64, kFlagPre64, kValMask64>(status, vb, 1);
      st_dev(status + vb, kFlagPre64 | (excl + tot));
    }
    s_excl = excl;
    if ((uint64_t)(vb + 1) * kScanTile >= (uint64_t)n) {  // the last workgroup knows P
      const uint64_t P = excl + tot;
      ctrl->num_pairs = P;
      ctrl->eff_pairs = P <= capacity ? P : 0u;
      if (user_num_pairs) *user_num_pairs = (int64_t)P;
    }
  }
  __syncthreads();
  const uint64_t excl = s_excl;
  // pairs [excl, excl + tot) belong to this workgroup; those at or past the capacity are dropped
  // (then P > capacity and no later kernel reads any pair)
  const uint32_t emit = excl >= capacity ? 0u : (uint32_t)std::min<uint64_t>(tot, capacity - excl);
  for (uint32_t j = tid; j < emit; j += kScanTile) {
    // owner: the first Gaussian whose inclusive count exceeds j (j < 2^30, below saturation)
    uint32_t lo = 0;
#pragma unroll
    for (uint32_t step = kScanTile / 2; step > 0; step >>= 1)
      if (s_incl[lo + step - 1] <= j) lo += step;
    const uint32_t local = j - (lo ? s_incl[lo - 1] : 0u);
    const uint32_t ww = (uint32_t)s_w[lo];
    const uint32_t row = local / ww, col = local - row * ww;
    const uint32_t t = (uint32_t)(s_y0[lo] + (int32_t)row) * (uint32_t)tiles_x + (uint32_t)s_x0[lo] + col;
    pkeys[excl + j] = t;
    pvals[excl + j] = s_g[lo];
    for (int p = 0; p < npass; ++p) atomicAdd(&s_hist[p][(t >> (8 * p)) & 0xFF], 1u);
  }
  __syncthreads();
  for (int p = 0; p < npass; ++p) {
    const uint32_t h = s_hist[p][tid];
    if (h) atomicAdd(&ctrl->hist_pair[p][tid], h);
  }
}

// ---------------------------------------------------------------------------------------------
// 6. per-tile ranges from the sorted 64-bit keys (the ranges were zeroed by k_bin_prep)
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ranges(const uint64_t* __restrict__ n_dev, const uint64_t* __restrict__ keys,
                                                uint32_t ntiles, uint32_t* __restrict__ ranges) {
  const uint64_t P = *n_dev;
  const uint64_t i = blockIdx.x * 256ull + threadIdx.x;
  if (i >= P) return;
  const uint32_t t = (uint32_t)(keys[i] >> 32);
  if (t >= ntiles) return;
  if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * t] = (uint32_t)i;
  if (i == P - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * t + 1] = (uint32_t)(i + 1);
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t count, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------------------------
// workspace layout: [ctrl | scan look-back | depth look-back | pair look-back] are zeroed by
// k_bin_prep; the rest is written before it is read
// ---------------------------------------------------------------------------------------------
struct BinLayout {
  size_t ctrl, scan_status, dstatus, pstatus, zero_end;
  size_t dhist, dkA, dvA, dkB, dvB, pkB, pvB, total;
  uint32_t nbN, nbS, nbCap;
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
  L.nbS = (uint32_t)((n + kScanTile - 1) / kScanTile);
  L.nbCap = (uint32_t)((cap + kSortTile - 1) / kSortTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, A);
    return at;
  };
  L.ctrl = take(sizeof(Ctrl));
  L.scan_status = take((size_t)L.nbS * 8);
  L.dstatus = take((size_t)4 * L.nbN * kRadix * 4);
  L.pstatus = take((size_t)L.npass * L.nbCap * kRadix * 4);
  L.zero_end = off;
  L.dhist = take((size_t)L.nbN * 4 * kRadix * 4);
  L.dkA = take((size_t)n * 4);
  L.dvA = take((size_t)n * 4);
  L.dkB = take((size_t)n * 4);
  L.dvB = take((size_t)n * 4);
  L.pkB = take((size_t)cap * 4);
  L.pvB = take((size_t)cap * 4);
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
                                     uint32_t* d_ids, uint32_t* d_tile_ranges, int64_t* d_num_pairs,
                                     int64_t* h_num_pairs, void* stream) {
  std::string why;
  if (n < 0) return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: n < 0");
  if (!valid_camera(cam, &why)) return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: " + why);
  if (!d_tile_ranges || pair_capacity < 0)
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL d_tile_ranges or capacity < 0");
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  if (ntiles > ((int64_t)1 << 24)) return set_error(GS_ERR_LIMIT, "gs_bin_and_sort: more than 2^24 tiles");
  if ((int64_t)n > (int64_t)kValMask || pair_capacity > (int64_t)kValMask)
    return set_error(GS_ERR_LIMIT, "gs_bin_and_sort: n or pair capacity above 2^30 - 1");
  if (pair_capacity > 0 && (!d_keys || !d_ids))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL d_keys/d_ids with capacity > 0");
  if (n > 0 && (!proj || !proj->d_depths || !proj->d_tiles_touched || !proj->d_means2d || !proj->d_radii))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: NULL projected record with n > 0");
  const BinLayout L = bin_layout(n, pair_capacity, cam);
  if (n > 0 && (!d_workspace || workspace_bytes < L.total))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: workspace smaller than gs_bin_workspace_bytes()");
  if (((reinterpret_cast<uintptr_t>(d_workspace) & 255) != 0) || ((reinterpret_cast<uintptr_t>(d_keys) & 7) != 0) ||
      ((reinterpret_cast<uintptr_t>(d_num_pairs) & 7) != 0))
    return set_error(GS_ERR_INVALID_ARG,
                     "gs_bin_and_sort: workspace must be 256-byte aligned, d_keys and d_num_pairs 8-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (h_num_pairs) *h_num_pairs = 0;
  if (n == 0) {
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((2 * ntiles + 255) / 256)), dim3(256), 0, s, d_tile_ranges,
                       (size_t)(2 * ntiles), 0u);
    if (d_num_pairs) hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, s, (uint32_t*)d_num_pairs, (size_t)2, 0u);
    return check_launch("gs_bin_and_sort");
  }
  char* ws = (char*)d_workspace;
  Ctrl* ctrl = (Ctrl*)(ws + L.ctrl);
  uint32_t *dkA = (uint32_t*)(ws + L.dkA), *dvA = (uint32_t*)(ws + L.dvA), *dkB = (uint32_t*)(ws + L.dkB),
           *dvB = (uint32_t*)(ws + L.dvB), *dhist = (uint32_t*)(ws + L.dhist);
  uint64_t* scan_status = (uint64_t*)(ws + L.scan_status);
  uint32_t* dstatus = (uint32_t*)(ws + L.dstatus);
  uint32_t* pstatus = (uint32_t*)(ws + L.pstatus);
  const size_t zero_words = (L.zero_end - L.ctrl) / 4;
  {
    // enough workgroups for the depth keys, and for zeroing about 32 words per thread
    const size_t zwords = zero_words + (size_t)(2 * ntiles);
    const size_t zblocks = (zwords + 32 * kSortThreads - 1) / (32 * kSortThreads);
    const unsigned blocks = (unsigned)std::max<size_t>(L.nbN, std::min<size_t>(zblocks, 2048));
    TimedScope ts("bin_prep", s);
    hipLaunchKernelGGL(k_bin_prep, dim3(blocks), dim3(kSortThreads), 0, s, n, proj->d_depths, proj->d_tiles_touched,
                       dkA, dvA, dhist, L.nbN, (uint32_t*)(ws + L.ctrl), zero_words, d_tile_ranges,
                       (size_t)(2 * ntiles));
  }
  // up to kDirectHistRows workgroups, each depth pass sums the per-workgroup histograms itself
  const bool direct_hist = L.nbN <= (uint32_t)kDirectHistRows;
  if (!direct_hist) {
    TimedScope ts("hist_reduce", s);
    hipLaunchKernelGGL(k_hist_reduce, dim3(4, (L.nbN + kReduceRows - 1) / kReduceRows), dim3(kRadix), 0, s, dhist,
                       L.nbN, ctrl);
  }
  for (int p = 0; p < 4; ++p) {
    const bool even = (p % 2) == 0;
    const uint32_t* hist = direct_hist ? dhist + p * kRadix : ctrl->hist_depth[p];
    TimedScope ts("depth_sort_pass", s);
    hipLaunchKernelGGL(k_onesweep<false>, dim3(L.nbN), dim3(kSortThreads), 0, s, even ? dkA : dkB, even ? dvA : dvB,
                       even ? dkB : dkA, even ? dvB : dvA, (uint64_t*)nullptr, (const uint32_t*)nullptr,
                       (uint32_t)n, (const uint64_t*)nullptr, 8 * p, 8, hist, direct_hist ? (int)L.nbN : 1,
                       4 * kRadix, dstatus + (size_t)p * L.nbN * kRadix, &ctrl->tickets[p]);
  }
  // ping-pong of the pair sort: A = d_keys viewed as two u32 arrays of pair_capacity, B = workspace
  uint32_t* kA = (uint32_t*)d_keys;
  uint32_t* vA = kA ? kA + pair_capacity : nullptr;
  uint32_t *kB = (uint32_t*)(ws + L.pkB), *vB = (uint32_t*)(ws + L.pvB);
  const bool emit_to_A = (L.npass % 2) == 0;
  const int32_t tiles_x = (cam->width + 15) / 16, tiles_y = (cam->height + 15) / 16;
  {
    TimedScope ts("scan_emit", s);
    hipLaunchKernelGGL(k_scan_emit, dim3(L.nbS), dim3(kScanTile), 0, s, n, dvA, proj->d_tiles_touched,
                       proj->d_means2d, proj->d_radii, tiles_x, tiles_y, emit_to_A ? kA : kB, emit_to_A ? vA : vB,
                       (uint64_t)pair_capacity, L.npass, scan_status, ctrl, d_num_pairs);
  }
  if (L.nbCap > 0) {
    bool in_A = emit_to_A;
    for (int p = 0; p < L.npass; ++p) {
      const int shift = 8 * p;
      const int bits = (L.tile_bits - shift) < 8 ? (L.tile_bits - shift) : 8;
      const bool last = p == L.npass - 1;
      uint32_t *ki = in_A ? kA : kB, *vi = in_A ? vA : vB;
      uint32_t *ko = in_A ? kB : kA, *vo = in_A ? vB : vA;
      TimedScope ts("pair_sort_pass", s);
      if (last) {
        hipLaunchKernelGGL(k_onesweep<true>, dim3(L.nbCap), dim3(kSortThreads), 0, s, ki, vi, (uint32_t*)nullptr,
                           d_ids, d_keys, (const uint32_t*)proj->d_depths, 0u, &ctrl->eff_pairs, shift, bits,
                           ctrl->hist_pair[p], 1, 0, pstatus + (size_t)p * L.nbCap * kRadix, &ctrl->tickets[4 + p]);
      } else {
        hipLaunchKernelGGL(k_onesweep<false>, dim3(L.nbCap), dim3(kSortThreads), 0, s, ki, vi, ko, vo,
                           (uint64_t*)nullptr, (const uint32_t*)nullptr, 0u, &ctrl->eff_pairs, shift, bits,
                           ctrl->hist_pair[p], 1, 0, pstatus + (size_t)p * L.nbCap * kRadix, &ctrl->tickets[4 + p]);
      }
      in_A = !in_A;
    }
    TimedScope ts("ranges", s);
    hipLaunchKernelGGL(k_ranges, dim3((unsigned)((pair_capacity + 255) / 256)), dim3(256), 0, s, &ctrl->eff_pairs,
                       d_keys, (uint32_t)ntiles, d_tile_ranges);
  }
  const gs_status st = check_launch("gs_bin_and_sort");
  if (st != GS_OK || !h_num_pairs) return st;
  uint64_t P = 0;
  if (hipMemcpyAsync(&P, &ctrl->num_pairs, sizeof(P), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return check_launch("gs_bin_and_sort: reading the pair count");
  *h_num_pairs = (int64_t)P;
  if ((int64_t)P > pair_capacity)
    return set_error(GS_ERR_CAPACITY, "gs_bin_and_sort: " + std::to_string(P) + " pairs exceed the capacity " +
                                          std::to_string(pair_capacity));
  return GS_OK;
}
