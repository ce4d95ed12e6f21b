// Binning: count, emit, sort and range of tile/Gaussian pairs.
//
// What is computed ("SplatRs: The Week the Gap Closed", section "Throughput: the tile
// rasterizer": project, count, emit, sort, range): for every drawn Gaussian i and every tile of
// its rectangle, the pair (key = tile << 32 | float_bits(depth_i), value = i), the pairs sorted
// by key with equal keys in ascending i, and the per-tile [start, end) ranges.
//
// How (MI355X design, not the pages'): a full 64-bit key sort would take 6 radix passes over the
// pairs. Here the depth part is settled once per Gaussian instead of once per pair:
//   1. k_bin_prep     depth keys (culled -> 0xFFFFFFFF), packed (count, first tile, width,
//                     height) rectangles, per-workgroup digit histograms of the four depth passes, and
//                     the zeroing of every counter, look-back word and
//                     tile range the later kernels rely on (no memset nodes, no host wait)
//   2. k_hist_reduce  the per-workgroup depth histograms summed (beyond 32 workgroups; below
//                     that each depth pass sums them itself)
//   3. 4 x k_onesweep stable LSD radix sort of the N Gaussians by depth bits; the first pass drops
//                     the culled ones (their key is 0xFFFFFFFF and the histograms leave them out),
//                     so the later passes, the scan and the emission see only the V drawn ones
//                     (a camera inside a large scene draws a tenth of it); extra workgroups of
//                     the first two passes count the pairs of every tile (they do not depend on
//                     the depth order) and turn the counts into the tile ranges and the
//                     tile-digit histograms of the pair sort
//   4. k_scan         single-pass prefix scan of the tile counts in depth order (4096 Gaussians
//                     per workgroup, wave-wide look-back): per Gaussian in depth order its first
//                     pair position, rectangle and id; per chunk of 4096 pair positions the
//                     Gaussian it starts in; the last workgroup publishes P
//   5. k_emit_sort    one workgroup per chunk of 4096 pair positions emits those (tile id, i)
//                     pairs into LDS, however the pairs spread over Gaussians (the nearest
//                     splats, first in depth order, cover thousands of tiles): the owner of each
//                     position is a max-scan of the markers that staged Gaussians leave at their
//                     first position; then it runs the first radix pass of the pairs on them
//   6. ceil(bits/8) - 1 x k_onesweep  the remaining stable LSD radix passes of the pairs by tile
//                     id (the tile-id bits split evenly over the passes); the last pass writes the
//                     64-bit key (tile << 32 | depth bits of i) and the id
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
// writes 12 and gathers 4). With 2 pair passes that is 8 + 16 + 24 = 48 B/pair, plus 64 B per
// Gaussian (prep and the first depth pass) and about 90 B per drawn Gaussian (three depth
// passes, the scan, the emission's records).
#include <algorithm>
#include <mutex>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kSortThreads = 1024;  // 16 waves: short per-wave ranking chains
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 4;
constexpr int kSortTile = kSortThreads * kSortItems;  // 4096 keys per workgroup
constexpr int kEmitThreads = 1024;
constexpr int kEmitWaves = kEmitThreads / 64;
constexpr int kScanItems = 4;
constexpr int kScanTile = kEmitThreads * kScanItems;  // 4096 Gaussians per scan workgroup
constexpr int kEmitPer = 4;
constexpr int kEmitChunk = kEmitThreads * kEmitPer;   // pair positions per emit workgroup
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
  uint64_t n_visible;    // drawn Gaussians (large frames: the depth sort's length after its first pass)
  uint32_t tickets[16];  // [0..3] depth passes, [4..6] pair passes, [7] scan, [8] scan workgroups done
  uint32_t hist_depth[4][kRadix];
  uint32_t hist_pair[3][kRadix];
};

// The lanes of the wave whose `bits`-bit digit equals this lane's (a 64-bit lane mask), from one
// ballot per bit: a lane whose bit is 1 keeps the ballot's lanes, one whose bit is 0 its
// complement. The flip mask makes that one xor-and per half of the mask.
template <int MAXBITS>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int bits, uint64_t m) {
  uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
#pragma unroll
  for (int b = 0; b < MAXBITS; ++b) {
    if (b < bits) {  // uniform
      const uint32_t bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      const uint32_t flip = bit - 1u;  // 0 keeps the ballot, all ones complements it
      lo &= (uint32_t)bb ^ flip;
      hi &= (uint32_t)(bb >> 32) ^ flip;
    }
  }
  return ((uint64_t)hi << 32) | lo;
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

// Exclusive sum over one value per thread of a 1024-thread workgroup; *total gets the sum. Two
// barriers; every thread calls it.
template <typename T>
__device__ __forceinline__ T block_excl_scan1024(T v, T* s_wsum, T* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T inc = wave_incl_scan<T>(v, lane);
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  T before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kSortWaves; ++w) {
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
                                                           const float* __restrict__ means2d,
                                                           const int32_t* __restrict__ radii, int32_t tiles_x,
                                                           int32_t tiles_y, uint4* __restrict__ rec,
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
  uint32_t k[kSortItems], t[kSortItems];
  float2 m[kSortItems];
  int2 r[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {  // all loads in flight before any is used
    const int idx = base + i * kSortThreads + tid;
    t[i] = idx < n ? tiles[idx] : 0u;
    const float z = idx < n ? depths[idx] : 0.0f;
    m[i] = idx < n ? *reinterpret_cast<const float2*>(means2d + 2 * idx) : make_float2(0.0f, 0.0f);
    r[i] = idx < n ? *reinterpret_cast<const int2*>(radii + 2 * idx) : make_int2(0, 0);
    k[i] = t[i] > 0 ? __float_as_uint(z) : 0xFFFFFFFFu;
  }
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const int idx = base + i * kSortThreads + tid;
    if (idx < n) {
      keys[idx] = k[i];
      vals[idx] = (uint32_t)idx;
      uint32_t tb = 0, w = 1, h = 0;
      if (t[i] > 0) {
        const TileRect rc = tile_rect(m[i].x, m[i].y, (float)r[i].x, (float)r[i].y, tiles_x, tiles_y);
        tb = (uint32_t)(rc.y0 * tiles_x + rc.x0);
        w = (uint32_t)(rc.x1 - rc.x0);
        h = (uint32_t)(rc.y1 - rc.y0);
      }
      rec[idx] = make_uint4(t[i], tb, w, h);
      if (t[i] > 0) {  // culled keys leave the depth sort in its first pass
#pragma unroll
        for (int p = 0; p < 4; ++p) atomicAdd(&s_hist[p][(k[i] >> (8 * p)) & 0xFF], 1u);
      }
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
constexpr int kReduceRows = 8;       // rows per workgroup: independent loads, many workgroups
constexpr int kDirectHistRows = 32;  // up to here each depth pass sums the rows itself
__global__ __launch_bounds__(kRadix) void k_hist_reduce(const uint32_t* __restrict__ dhist, uint32_t nbN, Ctrl* ctrl) {
  const int p = blockIdx.x, d = threadIdx.x;
  const uint32_t r0 = blockIdx.y * kReduceRows;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kReduceRows; ++i)
    if (r0 + i < nbN) s += dhist[((size_t)(r0 + i) * 4 + p) * kRadix + d];
  if (s) atomicAdd(&ctrl->hist_depth[p][d], s);
}

// ---------------------------------------------------------------------------------------------
// Pairs per tile, tile ranges and the tile-digit histograms of the pair sort. The count of pairs
// per tile does not depend on the depth order, so extra workgroups of the first two depth passes
// compute it while those passes sort: row y of a rectangle puts one pair on each tile of the run
// [a, a + w) of tile ids (with tight tiles the row's run [xs, xe) of tight_row), i.e. +1 at a
// and -1 at a + w of a difference array over the tiles
// (pass 0); one workgroup then prefix-sums it into per-tile counts, ranges and histograms
// (pass 1). The total of the counts is P, so that workgroup also knows whether P fits the
// capacity (else every range stays (0, 0)).
// ---------------------------------------------------------------------------------------------
struct TileCountArgs {
  const uint4* rec;     // (count, first tile, width, height) per Gaussian, id order (k_bin_prep)
  const float* means2d; // with tight: the ellipse of each Gaussian (tight_shape)
  const float* conics;
  const float* opac;
  int32_t tight;        // camera option tight_tiles: rows hold the tight runs, not the whole width
  int32_t n;
  int32_t tiles_x;
  uint32_t ntiles;
  uint32_t* tdiff;      // ntiles + 1 words, zeroed by k_bin_prep
  uint32_t* ranges;     // [ntiles, 2], zeroed by k_bin_prep
  uint32_t* plan;       // raster plan (optional; layout in gs_internal.h)
  uint64_t capacity;
  int npass;
  int pshift[3];        // the pair passes' digit shifts and widths (tile id bits split evenly)
  int pbits[3];
  uint32_t* hist_pair;  // [npass][256]
  // small frames: the difference array is the sum of tmat_rows rows, tmat_stride apart (one per
  // sorted block), and the finalizer writes every tile's range, (0, 0) included, since nothing
  // zeroed them
  const uint32_t* tmat;
  uint32_t tmat_rows;
  uint32_t tmat_stride;
  int32_t all_ranges;
};

constexpr uint32_t kMaxTmatRows = 9;  // the small-frame path's blocks
// Entry t of the difference array: the sum of the rows' entries, their loads all in flight.
__device__ __forceinline__ uint32_t tdiff_at(const TileCountArgs& a, uint32_t t) {
  if (!a.tmat) return a.tdiff[t];
  uint32_t v[kMaxTmatRows];
#pragma unroll
  for (uint32_t r = 0; r < kMaxTmatRows; ++r)
    v[r] = a.tmat[(size_t)(r < a.tmat_rows ? r : 0u) * a.tmat_stride + t];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t r = 0; r < kMaxTmatRows; ++r) sum += r < a.tmat_rows ? v[r] : 0u;
  return sum;
}
constexpr int kRowGaussians = 2048;  // Gaussians per row workgroup (two per lane)

// Row workgroup rb: Gaussians [2048 rb, 2048 (rb + 1)) of the id order, two per lane. A lane
// walks the rows of its own Gaussian when there are at most kOwnRows (tight rows: kOwnRowsTight)
// of them; the taller ones
// are walked by the whole wave, one Gaussian at a time (its rectangle read with readlane), so a
// screen-filling splat does not hold up its wave. The difference array is staged in LDS (`lds`,
// `lds_words` long) when it fits.
constexpr uint32_t kOwnRows = 8;
constexpr uint32_t kOwnRowsTight = 32;  // tight rows cost more each, the wave walk wastes more lanes
__device__ __forceinline__ TightShape tight_of(const TileCountArgs& a, uint32_t g) {
  const float2 m = *reinterpret_cast<const float2*>(a.means2d + 2 * (size_t)g);
  const float* c = a.conics + 3 * (size_t)g;
  return tight_shape(m.x, m.y, c[0], c[1], c[2], a.opac[g]);
}
// One Gaussian per lane (rectangle r = (count, first tile, width, height), id j; valid lanes
// only add): a lane walks its own rows when there are at most kOwnRows (tight: kOwnRowsTight);
// taller rectangles are walked by the whole wave, one at a time. Every lane of the wave calls it.
__device__ void tile_rows_item(const TileCountArgs& a, uint4 r, uint32_t j, bool valid, uint32_t* diff) {
  const int lane = threadIdx.x & 63;
  const uint32_t tx = (uint32_t)a.tiles_x;
  const uint32_t h = valid ? r.w : 0u;
  // with tight tiles each lane prepares its own Gaussian's ellipse once; the wave walk of a
  // tall one takes it from the owning lane
  TightShape own{};
  if (a.tight && h > 0) own = tight_of(a, j);
  const uint32_t own_max = a.tight ? kOwnRowsTight : kOwnRows;
  if (h <= own_max) {
    if (a.tight && h > 0) {
      const TightShape& ts = own;
      const int x0 = (int)(r.y % tx), y0 = (int)(r.y / tx);
      for (uint32_t y = 0; y < h; ++y) {
        const int2 sp = tight_row(ts, y0 + (int)y, x0, x0 + (int)r.z);
        if (sp.y > sp.x) {
          atomicAdd(&diff[(uint32_t)(y0 + (int)y) * tx + (uint32_t)sp.x], 1u);
          atomicSub(&diff[(uint32_t)(y0 + (int)y) * tx + (uint32_t)sp.y], 1u);
        }
      }
    } else {
      for (uint32_t y = 0; y < h; ++y) {
        atomicAdd(&diff[r.y + y * tx], 1u);
        atomicSub(&diff[r.y + y * tx + r.z], 1u);
      }
    }
  }
  uint64_t tall = __ballot(h > own_max);
  while (tall) {
    const int src = __builtin_ctzll(tall);
    tall &= tall - 1;
    const uint32_t hh = __builtin_amdgcn_readlane(h, src);
    const uint32_t tb = __builtin_amdgcn_readlane(r.y, src), w = __builtin_amdgcn_readlane(r.z, src);
    if (a.tight) {
      TightShape ts;
      ts.mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.mx), src));
      ts.my = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.my), src));
      ts.A = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.A), src));
      ts.B = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.B), src));
      ts.C = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.C), src));
      ts.D = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.D), src));
      ts.s2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.s2), src));
      ts.E = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own.E), src));
      ts.full = __builtin_amdgcn_readlane((int)own.full, src) != 0;
      const int x0 = (int)(tb % tx), y0 = (int)(tb / tx);
      for (uint32_t y = lane; y < hh; y += 64) {
        const int2 sp = tight_row(ts, y0 + (int)y, x0, x0 + (int)w);
        if (sp.y > sp.x) {
          atomicAdd(&diff[(uint32_t)(y0 + (int)y) * tx + (uint32_t)sp.x], 1u);
          atomicSub(&diff[(uint32_t)(y0 + (int)y) * tx + (uint32_t)sp.y], 1u);
        }
      }
    } else {
      for (uint32_t y = lane; y < hh; y += 64) {
        atomicAdd(&diff[tb + y * tx], 1u);
        atomicSub(&diff[tb + y * tx + w], 1u);
      }
    }
  }
}

__device__ void tile_rows(const TileCountArgs& a, uint32_t rb, uint32_t* lds, uint32_t lds_words) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool staged = a.ntiles + 1 <= lds_words;
  if (staged) {
    for (uint32_t t = tid; t <= a.ntiles; t += kSortThreads) lds[t] = 0;
    __syncthreads();
  }
  uint32_t* diff = staged ? lds : a.tdiff;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int64_t j = (int64_t)rb * kRowGaussians + wave * 128 + k * 64 + lane;
    const bool valid = j < a.n;
    const uint4 r = valid ? a.rec[j] : make_uint4(0u, 0u, 1u, 0u);
    tile_rows_item(a, r, (uint32_t)j, valid, diff);
  }
  if (staged) {
    __syncthreads();
    for (uint32_t t = tid; t <= a.ntiles; t += kSortThreads) {
      const uint32_t v = lds[t];
      if (v) atomicAdd(&a.tdiff[t], v);
    }
  }
}

// One workgroup, in steps of 10240 tiles held in LDS (one step up to 10240 tiles): thread tid
// takes tiles 1024 q + tid, so each row of 1024 tiles is loaded and stored contiguously. The
// difference array is scanned into per-tile counts and the counts into range starts, in place.
// A first sweep finds P (64 bits) and how many tiles fall in each count class (bit length of the
// count), per XCD list (plan_xcd). A second writes the ranges and the pair-sort histograms (when P
// fits), the processing order (each XCD's list heaviest class first, empty tiles last, so that
// the long raster workgroups start first; the lists interleaved so that a tile's slot runs on its
// XCD), and for each tile of two or more chunks of L its checkpoint slots and extra work items
// (chunks 1 ..). With one step the second sweep finds the starts still in LDS.
// The code is loops over rows rather than unrolled: it runs once per frame, on one compute unit,
// where straight-line code would wait on instruction fetch.
// Histogram digits above the lowest (shift s > 0) are constant over aligned runs of 2^s tiles: a
// run's count is the difference of the range starts at its ends, added with two LDS atomics.
__device__ __forceinline__ uint32_t count_class(uint32_t c) { return c ? 32u - (uint32_t)__clz(c) : 0u; }

// Lanes with the same key (BITS bits) share one LDS atomic on ctr[key]; returns a valid lane's
// place. Every lane of the wave calls it.
template <int BITS>
__device__ __forceinline__ uint32_t wave_key_slot(bool valid, uint32_t key, uint32_t* ctr, int lane) {
  const uint64_t m = match_digit<BITS>(key, BITS, __ballot(valid));
  const int leader = __builtin_ctzll(m | (1ull << 63));
  uint32_t base = 0;
  if (valid && lane == leader) base = atomicAdd(&ctr[key], (uint32_t)__popcll(m));
  base = __shfl(base, leader, 64);
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  return base + (uint32_t)__popcll(m & lt);
}

// The wave's lanes take v consecutive units each of the LDS counter *ctr, in lane order, with one
// atomic for the wave (none when the wave takes nothing); returns the lane's first unit. Every
// lane of the wave calls it.
__device__ __forceinline__ uint32_t wave_take(uint32_t v, uint32_t* ctr, int lane);
// Work items (t, 1 .. n) of a tile from position x0 on (two words each): a lane writes its own
// tile's when they are few, the wave together (one tile at a time) for longer lists. Every lane of
// the wave calls it.
__device__ __forceinline__ void write_items(uint32_t n, uint32_t x0, uint32_t t, uint32_t* items, int lane) {
  constexpr uint32_t kOwnItems = 8;
  if (n <= kOwnItems)
    for (uint32_t j = 0; j < n; ++j) {
      items[2 * (x0 + j)] = t;
      items[2 * (x0 + j) + 1] = j + 1u;
    }
  uint64_t mm = __ballot(n > kOwnItems);
  while (mm) {
    const int src = __builtin_ctzll(mm);
    mm &= mm - 1;
    const uint32_t n1 = (uint32_t)__builtin_amdgcn_readlane((int)n, src);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x0, src);
    const uint32_t tt = (uint32_t)__builtin_amdgcn_readlane((int)t, src);
    for (uint32_t j = (uint32_t)lane; j < n1; j += 64) {
      items[2 * (b + j)] = tt;
      items[2 * (b + j) + 1] = j + 1u;
    }
  }
}

// DPP lane shifts within rows of 16 lanes (row_shr) and row broadcasts (row_bcast); lanes whose
// source lies outside the row read 0, lanes of rows outside ROWMASK are left as they are.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWMASK, 0xf, true);
}
// Inclusive sum within each row of 16 lanes.
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(v);  // row_shr:1
  v += dpp_u32<0x112, 0xf>(v);  // row_shr:2
  v += dpp_u32<0x114, 0xf>(v);  // row_shr:4
  v += dpp_u32<0x118, 0xf>(v);  // row_shr:8
  return v;
}
// Inclusive sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v = row16_incl_scan(v);
  v += dpp_u32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint32_t wave_take(uint32_t v, uint32_t* ctr, int lane) {
  const uint32_t inc = wave_incl_scan_dpp(v);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  uint32_t base = 0;
  if (tot != 0u) {  // wave-uniform
    if (lane == 0) base = atomicAdd(ctr, tot);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
  }
  return base + inc - v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

constexpr int kFinRows = 10;
constexpr uint32_t kFinStep = kSortThreads * kFinRows;
constexpr uint32_t kFinAuxWords = 8 * kRadix;  // histograms, classes, scan partials
constexpr uint32_t kFinClasses = 33;           // count classes 0 (empty) .. 32
constexpr uint32_t kFinKeys = kXcds * kFinClasses;  // (XCD, class): key x * 33 + class, 9 bits
constexpr uint32_t kFinMisc = 16;
static_assert(kFinKeys <= 512, "the (XCD, class) key takes 9 bits");
static_assert(3 * kRadix + 2 * kFinKeys + kFinMisc + 17 * kFinRows <= kFinAuxWords, "finalizer auxiliary words overflow");

// Exclusive scan, in place, of `rows` rows of 1024 values in LDS (s[1024 q + tid] in thread
// tid), offset by carry; returns the sum (mod 2^32). Every thread calls it; it ends with a
// barrier, after which any thread may read any element.
__device__ uint32_t lds_rows_scan(uint32_t* s, int rows, uint32_t carry, uint32_t* s_wt, uint32_t* s_rt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll 1
  for (int q = 0; q < rows; ++q) {
    uint32_t* p = s + q * kSortThreads + tid;
    const uint32_t v = *p;
    const uint32_t inc = wave_incl_scan_dpp(v);
    *p = inc - v;
    if (lane == 63) s_wt[q * kSortWaves + wave] = inc;
  }
  __syncthreads();
  if (tid < rows * kSortWaves) {  // a 16-lane row per row of tiles: the scan over its waves
    const uint32_t v = s_wt[tid];
    const uint32_t inc = row16_incl_scan(v);
    s_wt[tid] = inc - v;
    if ((tid & (kSortWaves - 1)) == kSortWaves - 1) s_rt[tid / kSortWaves] = inc;
  }
  __syncthreads();
  uint32_t before = carry;
#pragma unroll 1
  for (int q = 0; q < rows; ++q) {
    s[q * kSortThreads + tid] += before + s_wt[q * kSortWaves + wave];
    before += s_rt[q];
  }
  __syncthreads();
  return before - carry;
}

__device__ void tile_finalize(const TileCountArgs& a, uint32_t* lds, uint32_t lds_words) {
  __shared__ unsigned long long s_p64;
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* aux = lds + (lds_words - kFinAuxWords);
  uint32_t(*s_hist)[kRadix] = reinterpret_cast<uint32_t(*)[kRadix]>(aux);  // rows 0-2: histograms
  uint32_t* s_cls = aux + 3 * kRadix;  // tiles per (XCD, count class)
  uint32_t* s_cur = s_cls + kFinKeys;  // next place in the XCD's list per (XCD, class)
  // [0] extra work items, [1] checkpoint slots, [2] split chunks, [3] tail slots, [8 + x] the
  // length of XCD x's list
  uint32_t* s_misc = s_cur + kFinKeys;
  uint32_t* s_wt = s_misc + kFinMisc;  // kFinRows x 16 scan partials
  uint32_t* s_rt = s_wt + 16 * kFinRows;  // kFinRows row sums
  uint32_t* s = lds;                   // the step's tiles
  const bool one_step = a.ntiles <= kFinStep;
  if (tid < kRadix)
    for (int k = 0; k < a.npass; ++k) s_hist[k][tid] = 0;
  if (tid < (int)(2 * kFinKeys + kFinMisc)) s_cls[tid] = 0;  // classes, cursors, misc
  if (tid == 0) s_p64 = 0;
  __syncthreads();
  uint64_t P = 0;
  uint32_t P32 = 0, L = kPlanMinChunk, lbits = 7;  // L = 2^lbits
  uint32_t mlist = 0;                                // the shortest XCD list
  const uint32_t tiles_x = (uint32_t)a.tiles_x;
  static_assert(kPlanMinChunk == 128u, "lbits starts at log2 of the minimum chunk");
  bool fits = false;
#pragma unroll 1
  for (int sweep = 0; sweep < 2; ++sweep) {
    if (sweep == 1 && !fits && !a.plan && !a.all_ranges) break;
    uint32_t carry_d = 0, carry_c = 0;
#pragma unroll 1
    for (uint32_t cb = 0; cb < a.ntiles; cb += kFinStep) {
      const uint32_t m = a.ntiles - cb < kFinStep ? a.ntiles - cb : kFinStep;  // tiles in the step
      const int rows = (int)((m + kSortThreads - 1) / kSortThreads);
      uint32_t step_end = P32;  // the start after the step's last tile
      if (sweep == 0 || !one_step) {
        __syncthreads();  // the previous step's reads of s (neighbours included) are done
        if (a.tmat) {  // a tile's difference sums the blocks' rows: two rows' loads in flight together
#pragma unroll
          for (int q = 0; q < kFinRows; q += 2) {
            const uint32_t i0 = (uint32_t)(q * kSortThreads + tid), i1 = i0 + kSortThreads;
            const uint32_t v0 = (q < rows && i0 < m) ? tdiff_at(a, cb + i0) : 0u;
            const uint32_t v1 = (q + 1 < rows && i1 < m) ? tdiff_at(a, cb + i1) : 0u;
            if (q < rows) s[i0] = v0;
            if (q + 1 < rows) s[i1] = v1;
          }
        } else {  // every row's load in flight together
          uint32_t v[kFinRows];
#pragma unroll
          for (int q = 0; q < kFinRows; ++q) {
            const uint32_t i = (uint32_t)(q * kSortThreads + tid);
            v[q] = (q < rows && i < m) ? a.tdiff[cb + i] : 0u;
          }
#pragma unroll
          for (int q = 0; q < kFinRows; ++q)
            if (q < rows) s[q * kSortThreads + tid] = v[q];
        }
        // counts: the inclusive prefix of the differences = the next tile's exclusive one
        const uint32_t dtot = lds_rows_scan(s, rows, carry_d, s_wt, s_rt);
        carry_d += dtot;
        uint32_t c[kFinRows];
#pragma unroll
        for (int q = 0; q < kFinRows; ++q) {
          const uint32_t i = (uint32_t)(q * kSortThreads + tid);
          c[q] = (q < rows && i < m) ? (i + 1 < m ? s[i + 1] : carry_d) : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kFinRows; ++q)
          if (q < rows) s[q * kSortThreads + tid] = c[q];
        if (sweep == 0) {
          uint64_t c64 = 0;
#pragma unroll 1
          for (int q = 0; q < rows; ++q) {
            const uint32_t i = (uint32_t)(q * kSortThreads + tid);
            const uint32_t cq = s[i];  // this thread's own entry (0 past the step)
            c64 += cq;
            wave_key_slot<9>(i < m, plan_xcd(cb + i, tiles_x) * kFinClasses + count_class(cq), s_cls, lane);
          }
          c64 = wave_sum_u64(c64);
          if (lane == 0) atomicAdd(&s_p64, (unsigned long long)c64);
        }
        // range starts (mod 2^32: used only when P fits, < 2^30)
        carry_c += lds_rows_scan(s, rows, carry_c, s_wt, s_rt);
        step_end = carry_c;
      }
      if (sweep == 0) continue;
#pragma unroll 1
      for (int q = 0; q < rows; ++q) {
        const uint32_t i = (uint32_t)(q * kSortThreads + tid), t = cb + i;
        const bool valid = i < m;
        const uint32_t st = valid ? s[i] : 0u;
        const uint32_t c = (valid && fits) ? (i + 1 < m ? s[i + 1] : step_end) - st : 0u;
        if (c) {
          a.ranges[2 * t] = st;
          a.ranges[2 * t + 1] = st + c;
          atomicAdd(&s_hist[0][t & ((1u << a.pbits[0]) - 1u)], c);
        } else if (valid && a.all_ranges) {
          a.ranges[2 * t] = 0u;
          a.ranges[2 * t + 1] = 0u;
        }
        if (valid && fits) {
          // a run of 2^shift_k tiles starting at t: its digit-k count starts at -start(t) and
          // the previous run's gets start(t)
          for (int k = 1; k < a.npass; ++k) {
            const uint32_t dm = (1u << a.pbits[k]) - 1u;
            if ((t & ((1u << a.pshift[k]) - 1u)) == 0u) {
              atomicSub(&s_hist[k][(t >> a.pshift[k]) & dm], st);
              if (t) atomicAdd(&s_hist[k][((t - 1u) >> a.pshift[k]) & dm], st);
            }
          }
        }
        if (!a.plan) continue;
        // the tile's place in its XCD's list; the lists interleave (slot 8 place + x) up to the
        // shortest one's length, the longer lists' rest take the slots after that. The places of a
        // list cover [0, its length) and the rest [8 mlist, ntiles): every valid slot is below ntiles
        const uint32_t x = plan_xcd(t, tiles_x);
        const uint32_t place = wave_key_slot<9>(valid, x * kFinClasses + count_class(c), s_cur, lane);
        const bool rest = valid && place >= mlist;
        const uint32_t rslot = wave_take(rest ? 1u : 0u, &s_misc[3], lane);
        const uint32_t slot = rest ? kXcds * mlist + rslot : kXcds * place + x;
        if (valid && slot < a.ntiles) a.plan[kPlanOrder + slot] = t;
        // a tile of two or more chunks: its checkpoint slots and extra work items (chunks 1 ..); a
        // tile the training forward splits: its blended chunks after the first, in order (c is 0
        // for lanes past the step and on overflow)
        const uint32_t nch = (c + L - 1u) >> lbits;
        const bool multi = nch >= 2u;
        const uint32_t nb = plan_split_pow2(c, lbits) ? plan_blended_chunks_pow2(c, lbits) : 1u;
        const uint32_t sb = wave_take(multi ? nch : 0u, &s_misc[1], lane);
        const uint32_t xb = wave_take(multi ? nch - 1u : 0u, &s_misc[0], lane);
        const uint32_t fb = wave_take(nb - 1u, &s_misc[2], lane);
        if (multi) a.plan[kPlanOrder + a.ntiles + t] = sb;
        write_items(multi ? nch - 1u : 0u, xb, t, a.plan + kPlanOrder + 2 * a.ntiles, lane);
        write_items(nb - 1u, fb, t, a.plan + kPlanOrder + 2 * a.ntiles + 2 * kPlanMaxChunks, lane);
      }
    }
    if (sweep == 0) {
      __syncthreads();  // every wave's class counts and count sums are in
      P = s_p64;
      P32 = carry_c;
      fits = P <= a.capacity;
      if (fits)
        while ((uint64_t)L * kPlanMaxChunks < P) {
          L <<= 1;
          ++lbits;
        }
      if (tid < (int)kXcds) {
        // XCD tid's list, heaviest class first; on overflow every tile is empty for the raster
        // calls: all in class 0
        uint32_t place = 0;
        for (int c = (int)kFinClasses - 1; c >= 0; --c) {
          const uint32_t k = (uint32_t)tid * kFinClasses + (uint32_t)c;
          s_cur[k] = fits ? place : 0u;
          place += s_cls[k];
        }
        s_misc[8 + tid] = place;
      }
      __syncthreads();
      mlist = s_misc[8];
      for (uint32_t x = 1; x < kXcds; ++x) mlist = min(mlist, s_misc[8 + x]);
    }
  }
  if (tid == 0 && fits)  // the last run ends at P
    for (int k = 1; k < a.npass; ++k)
      atomicAdd(&s_hist[k][((a.ntiles - 1u) >> a.pshift[k]) & ((1u << a.pbits[k]) - 1u)], (uint32_t)P);
  __syncthreads();
  if (tid < kRadix && fits)
    for (int k = 0; k < a.npass; ++k) a.hist_pair[k * kRadix + tid] = s_hist[k][tid];
  if (a.plan && tid == 0) {
    a.plan[kPlanChunk] = L;
    a.plan[kPlanExtra] = s_misc[0];
    a.plan[kPlanCheckpoints] = s_misc[1];
    a.plan[kPlanSplit] = s_misc[2];
  }
}

// ---------------------------------------------------------------------------------------------
// 3/6. one stable LSD radix pass over `bits` (<= 8) bits at `shift` (Onesweep-style)
// The element count is *n_dev when given (pairs: grid sized by the capacity), else n_host. The
// pass's digit histogram is the sum of `hist_parts` rows of 256 counts, `hist_stride` apart.
// ---------------------------------------------------------------------------------------------
// EXTRA: 0 none; 1 the last `n_extra` workgroups are tile-row workgroups; 2 the last one is the
// tile-count finalizer (see above). ITEMS keys per lane: a workgroup sorts 1024 ITEMS keys
// (4 keeps the ranking chains short for small inputs; 8 halves the workgroups, and so the
// look-back traffic, for large ones).
// Eight waves per SIMD (two 1024-thread workgroups per compute unit) need at most 64 VGPRs and
// about 80 SGPRs; the scalar registers are the tighter limit, so the target is spelled out.
// The part of a radix pass after the load, for one tile of 1024 ITEMS keys starting at `base`
// (ticket vb): item i of lane l of wave w is element base + 64 ITEMS w + 64 i + l (valid below n).
// Ranks the keys with wave ballots (stable), publishes the tile's digit counts, stages the keys
// in LDS in local sorted order, resolves the digits' global offsets by decoupled look-back and
// writes the keys out with consecutive threads. s_mem (2 TILE words) must hold zeroed per-wave
// digit counts in its first 16 x 256 words; h is this thread's digit count of the pass (threads
// below 256). Every thread calls it.
// DROP: keys equal to kCulledKey (culled Gaussians) are left out: the pass writes the other keys,
// densely, and its workgroup with ticket 0 stores their number (the sum of the pass's histogram,
// which does not count them) to *n_kept.
constexpr uint32_t kCulledKey = 0xFFFFFFFFu;
template <bool FINAL, int ITEMS, bool DROP = false>
__device__ __forceinline__ void radix_tile(uint32_t (&k)[ITEMS], uint32_t (&v)[ITEMS], uint32_t n, uint32_t base,
                                           uint32_t vb, int shift, int bits, uint32_t h, uint32_t* s_mem,
                                           uint32_t* s_dpre, uint32_t* s_goff, uint32_t* s_wsum,
                                           uint32_t* __restrict__ status, uint32_t* __restrict__ keys_out,
                                           uint32_t* __restrict__ vals_out, uint64_t* __restrict__ out_keys64,
                                           const uint32_t* __restrict__ depth_bits,
                                           uint64_t* __restrict__ n_kept = nullptr) {
  constexpr int TILE = kSortThreads * ITEMS;
  uint32_t* s_keys = s_mem;
  uint32_t* s_vals = s_mem + TILE;
  uint32_t (*s_wcnt)[kRadix] = reinterpret_cast<uint32_t (*)[kRadix]>(s_mem);  // count, then offset
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t mask = (1u << bits) - 1u;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t rank[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * ITEMS + i * 64 + lane);
    const bool valid = idx < n && (!DROP || k[i] != kCulledKey);
    const uint32_t d = (k[i] >> shift) & mask;
    const uint64_t m = match_digit<8>(d, bits, __ballot(valid));
    const uint32_t r = (uint32_t)__popcll(m & lt_mask);
    uint32_t pre = 0;
    if (valid) pre = s_wcnt[wave][d];
    rank[i] = pre + r;
    // keep the rank in one register from here on (left to itself the compiler keeps the
    // 64-bit match mask alive until the scatter, and the extra registers halve occupancy)
    asm volatile("" : "+v"(rank[i]));
    if (valid && r == 0) s_wcnt[wave][d] = pre + (uint32_t)__popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();

  // ---- per digit (threads below 2^bits): wave offsets, tile total, publish the aggregate ----
  const int radix = 1 << bits;
  uint32_t tot = 0;
  if (tid < radix) {
    // four waves' counts at a time: the keys, values and ranks are still live
#pragma unroll 4
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = s_wcnt[w][tid];
      s_wcnt[w][tid] = tot;
      tot += c;
    }
    st_dev(status + (size_t)vb * kRadix + tid, (vb == 0 ? kFlagPre : kFlagAgg) | tot);
  }
  uint32_t htot, ttot;
  const uint32_t bucket_excl = block_excl_scan256<uint32_t>(h, s_wsum, &htot);
  const uint32_t dpre = block_excl_scan256<uint32_t>(tot, s_wsum, &ttot);
  if (tid < kRadix) s_dpre[tid] = dpre;  // 0 past the pass's digits
  if (DROP && vb == 0 && tid == 0) st_dev(n_kept, (uint64_t)htot);
  __syncthreads();

  // ---- scatter to LDS in local sorted order (it needs no look-back, and frees the registers
  // of the keys before the look-back's loads are in flight) ----
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t d = (k[i] >> shift) & mask;
    rank[i] += s_dpre[d] + s_wcnt[wave][d];  // the local position
  }
  __syncthreads();  // the digit counts are dead: their LDS takes keys
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * ITEMS + i * 64 + lane);
    if (idx < n && (!DROP || k[i] != kCulledKey)) {
      s_keys[rank[i]] = k[i];
      s_vals[rank[i]] = v[i];
    }
  }
  // ---- look back for the digits' global offsets, then out with consecutive threads ----
  if (tid < radix) {
    uint32_t excl = 0;
    if (vb > 0) {
      excl = look_back<8, uint32_t, ~kValMask, kFlagPre, kValMask>(status + tid, vb, kRadix);
      st_dev(status + (size_t)vb * kRadix + tid, kFlagPre | (excl + tot));
    }
    s_goff[tid] = bucket_excl + excl - dpre;
  }
  __syncthreads();
  // the tile's keys in LDS: all of its range, or with DROP the kept ones (the digit totals' sum)
  const uint32_t count = DROP ? ttot : ((n - base < (uint32_t)TILE) ? (n - base) : (uint32_t)TILE);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
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

template <bool FINAL, int EXTRA, int ITEMS>
__global__ __launch_bounds__(kSortThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_onesweep(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, uint64_t* __restrict__ out_keys64, const uint32_t* __restrict__ depth_bits,
    uint32_t n_host, const uint64_t* __restrict__ n_dev, int shift, int bits, const uint32_t* __restrict__ hist,
    int hist_parts, int hist_stride, uint32_t* __restrict__ status, uint32_t* __restrict__ ticket,
    uint32_t n_extra, TileCountArgs targs, uint64_t* __restrict__ n_kept) {
  constexpr int TILE = kSortThreads * ITEMS;
  // the per-wave digit counts share LDS with the staged keys (they are dead by then), so a
  // workgroup of 8 keys per lane takes 64 KB and two fit on a compute unit; the extra
  // workgroups of the depth passes get 48 KB
  constexpr uint32_t kLdsWords = (EXTRA != 0 && 2 * TILE < 12288) ? 12288u : 2u * TILE;
  static_assert(kSortWaves * kRadix <= 2 * TILE, "digit counts must fit in the key staging");
  // the finalizer's step of tiles and its auxiliary words (histograms, classes, scan partials)
  // are disjoint parts of s_mem
  static_assert(EXTRA != 2 || kFinStep + kFinAuxWords <= kLdsWords, "finalizer LDS layout overlaps");
  __shared__ uint32_t s_mem[kLdsWords];
  uint32_t (*s_wcnt)[kRadix] = reinterpret_cast<uint32_t (*)[kRadix]>(s_mem);  // count, then offset
  __shared__ uint32_t s_dpre[kRadix];
  __shared__ uint32_t s_goff[kRadix];
  __shared__ uint32_t s_wsum[kSortWaves];
  __shared__ uint32_t s_vb;

  if (EXTRA != 0 && blockIdx.x >= gridDim.x - n_extra) {  // workgroup-uniform
    if (EXTRA == 1) tile_rows(targs, blockIdx.x - (gridDim.x - n_extra), s_mem, kLdsWords);
    if (EXTRA == 2) tile_finalize(targs, s_mem, kLdsWords);
    return;
  }
  const uint32_t n = n_dev ? (uint32_t)*n_dev : n_host;
  if ((uint64_t)blockIdx.x * TILE >= n) return;  // workgroup-uniform: idle workgroups take no ticket
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_vb = atomicAdd(ticket, 1u);
  for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  // exactly ceil(n / 4096) workgroups take tickets, so every ticket has base < n
  const uint32_t vb = s_vb;
  const uint32_t base = vb * (uint32_t)TILE;
  if (base >= n) return;  // unreachable with a zeroed ticket; guards a stale one
  // ---- load (wave-striped: wave w owns [base + 256 w, base + 256 (w + 1))) ----
  uint32_t k[ITEMS], v[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t idx = base + (uint32_t)(wave * 64 * ITEMS + i * 64 + lane);
    const bool valid = idx < n;
    k[i] = valid ? keys_in[idx] : 0u;
    v[i] = valid ? vals_in[idx] : 0u;
  }
  // the pass's histogram, read while the keys arrive: the sum of hist_parts rows, four threads per
  // digit each taking every fourth row, combined in the (not yet used) value staging of s_mem
  uint32_t h = 0;
  if (hist_parts == 1) {
    if (tid < kRadix) h = hist[tid];
  } else {
    uint32_t part = 0;
    for (int r = tid >> 8; r < hist_parts; r += kSortThreads / kRadix) part += hist[(size_t)r * hist_stride + (tid & (kRadix - 1))];
    uint32_t* s_part = s_mem + TILE;
    s_part[tid] = part;
    __syncthreads();
    if (tid < kRadix) {
#pragma unroll
      for (int q = 0; q < kSortThreads / kRadix; ++q) h += s_part[q * kRadix + tid];
    }
  }
  // the first depth pass (the one with the tile-row workgroups) drops the culled Gaussians
  radix_tile<FINAL, ITEMS, EXTRA == 1>(k, v, n, base, vb, shift, bits, h, s_mem, s_dpre, s_goff, s_wsum, status,
                                       keys_out, vals_out, out_keys64, depth_bits, n_kept);
}

// ---------------------------------------------------------------------------------------------
// 4. exclusive scan of tiles_touched in depth order (single pass, decoupled look-back)
// ---------------------------------------------------------------------------------------------
// Scan over one value per thread of a 1024-thread workgroup with an associative OP: returns the
// exclusive prefix (identity for thread 0); *total gets the reduction. Two barriers.
template <typename T, typename OP>
__device__ __forceinline__ T block_scan1024(T v, T identity, T* s_wsum, T* total, OP op) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  T inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T t = __shfl_up(inc, off, 64);
    if (lane >= off) inc = op(inc, t);
  }
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  T before = identity, all = identity;
#pragma unroll
  for (int w = 0; w < kEmitWaves; ++w) {
    const T x = s_wsum[w];
    if (w < wave) before = op(before, x);
    all = op(all, x);
  }
  __syncthreads();
  *total = all;
  const T ex = __shfl_up(inc, 1, 64);
  return op(before, lane == 0 ? identity : ex);
}

// Workgroup vb scans Gaussians [4096 vb, 4096 (vb + 1)) of the depth order (four consecutive per
// thread). It writes, in depth order, the record (first pair position, first tile, rect width,
// Gaussian id) of each, and for every pair chunk (kEmitChunk positions) that starts inside one of
// its Gaussians' runs, that Gaussian's depth index into chunk_first. The last workgroup
// publishes P.
__global__ __launch_bounds__(kEmitThreads) void k_scan(int32_t n_all, const uint64_t* __restrict__ n_drawn,
                                                       const uint32_t* __restrict__ sorted_ids,
                                                       const uint4* __restrict__ rec, uint4* __restrict__ drec,
                                                       uint32_t* __restrict__ chunk_first, uint64_t capacity,
                                                       uint64_t* __restrict__ status, Ctrl* ctrl,
                                                       int64_t* __restrict__ user_num_pairs) {
  __shared__ uint64_t s_wsum[kEmitWaves];
  __shared__ uint32_t s_vb;
  __shared__ uint64_t s_excl;
  // the depth order holds the drawn Gaussians only; workgroup 0 always runs, so P is published
  // also when none is drawn, and the idle ones take no ticket
  const int n = (int)min((uint64_t)n_all, *n_drawn);
  if (blockIdx.x > 0 && (int64_t)blockIdx.x * kScanTile >= n) return;  // workgroup-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_vb = atomicAdd(&ctrl->tickets[7], 1u);
  __syncthreads();
  const uint32_t vb = s_vb;
  uint4 r[kScanItems];
  uint32_t g[kScanItems];
  uint64_t sum = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const int j = (int)vb * kScanTile + tid * kScanItems + i;
    g[i] = j < n ? sorted_ids[j] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) r[i] = rec[g[i]];  // g = 0 past n: a valid index, unused
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const int j = (int)vb * kScanTile + tid * kScanItems + i;
    if (j >= n) r[i] = make_uint4(0u, 0u, 1u, 0u);
    sum += r[i].x;
  }
  uint64_t tot;
  const uint64_t texcl = block_scan1024<uint64_t>(sum, 0ull, s_wsum, &tot,
                                                   [](uint64_t a, uint64_t b) { return a + b; });
  // ---- publish, look back (wave 0: 64 predecessors per round), publish the prefix ----
  if (wave == 0) {
    if (lane == 0) st_dev(status + vb, (vb == 0 ? kFlagPre64 : kFlagAgg64) | tot);
    uint64_t excl = 0;
    int64_t j = (int64_t)vb - 1;
    while (j >= 0) {
      const int64_t p = j - lane;
      const uint64_t st = p >= 0 ? ld_dev(status + p) : kFlagPre64;  // below tile 0: never consumed
      const uint64_t fl = st & ~kValMask64;
      const uint64_t notready = __ballot(fl == 0), pre = __ballot(fl == kFlagPre64);
      const int first_nr = notready ? __builtin_ctzll(notready) : 64;
      const int first_pre = pre ? __builtin_ctzll(pre) : 64;
      const int take = first_pre < first_nr ? first_pre + 1 : first_nr;  // words consumed by this pass
      uint64_t v = lane < take ? (st & kValMask64) : 0ull;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      excl += v;
      if (first_pre < first_nr) break;
      j -= take;
      if (take == 0) __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      if (vb > 0) st_dev(status + vb, kFlagPre64 | (excl + tot));
      s_excl = excl;
      if ((uint64_t)(vb + 1) * kScanTile >= (uint64_t)n) {  // the last workgroup knows P
        const uint64_t P = excl + tot;
        ctrl->num_pairs = P;
        ctrl->eff_pairs = P <= capacity ? P : 0u;
        if (user_num_pairs) *user_num_pairs = (int64_t)P;
      }
    }
  }
  __syncthreads();
  uint64_t o = s_excl + texcl;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const int j = (int)vb * kScanTile + tid * kScanItems + i;
    if (j < n) {
      drec[j] = make_uint4(o < 0xFFFFFFFFull ? (uint32_t)o : 0xFFFFFFFFu, r[i].y, r[i].z, g[i]);
      const uint64_t end = o + r[i].x;
      for (uint64_t c = (o + kEmitChunk - 1) / kEmitChunk * kEmitChunk; c < end && c < capacity; c += kEmitChunk)
        chunk_first[c / kEmitChunk] = (uint32_t)j;
    }
    o += r[i].x;
  }
}

// ---------------------------------------------------------------------------------------------
// 5+6. emission fused with the first pair pass: the workgroup with ticket c emits pair positions
// [4096 c, 4096 (c + 1)) into LDS, each position's owner found by a max-scan over the staged
// Gaussians' first positions, then sorts them by the pass's digit and scatters them to the
// pass's output. The pass's digit histogram comes from the tile-count finalizer, so the pairs
// need not round-trip through memory before their first pass.
// ---------------------------------------------------------------------------------------------
constexpr int kFuseWindow = 1024;  // Gaussians staged per emission round (one per thread)
template <bool FINAL>
__global__ __launch_bounds__(kSortThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_emit_sort(
    const uint64_t* __restrict__ n_dev, int32_t n_all, const uint64_t* __restrict__ n_drawn,
    const uint4* __restrict__ drec,
    const uint32_t* __restrict__ chunk_first, int32_t tiles_x, int shift, int bits,
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ status, uint32_t* __restrict__ ticket,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint64_t* __restrict__ out_keys64,
    const uint32_t* __restrict__ depth_bits, TileCountArgs targs) {
  constexpr int ITEMS = 4, TILE = kSortThreads * ITEMS;
  static_assert(TILE == kEmitChunk && kEmitThreads == kSortThreads, "one emission chunk per sort tile");
  // the depth-ordered records: n_all, or (large frames) the drawn Gaussians only
  const int32_t n = n_drawn ? (int32_t)min((uint64_t)n_all, *n_drawn) : n_all;
  static_assert(kFuseWindow == kSortThreads, "one staged Gaussian per thread");
  __shared__ uint32_t s_mem[2 * TILE];  // the emitted pairs (keys, values), then the sort's staging
  __shared__ uint32_t s_owner[TILE];
  __shared__ uint32_t s_off[kFuseWindow];
  __shared__ uint32_t s_tb[kFuseWindow];
  __shared__ uint32_t s_w[kFuseWindow];
  __shared__ uint32_t s_g[kFuseWindow];
  __shared__ uint32_t s_dpre[kRadix];
  __shared__ uint32_t s_goff[kRadix];
  __shared__ uint32_t s_wsum[kSortWaves];
  __shared__ uint32_t s_vb;
  const uint64_t P = *n_dev;
  if ((uint64_t)blockIdx.x * TILE >= P) return;  // workgroup-uniform: idle workgroups take no ticket
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_vb = atomicAdd(ticket, 1u);
  __syncthreads();
  const uint32_t vb = s_vb;
  const uint64_t cs = (uint64_t)vb * TILE;
  if (cs >= P) return;  // unreachable with a zeroed ticket; guards a stale one
  const uint32_t ce = (uint32_t)(P - cs < (uint64_t)TILE ? P - cs : (uint64_t)TILE);
  uint32_t* s_pk = s_mem;
  uint32_t* s_pv = s_mem + TILE;

  // ---- emission of positions [cs, cs + ce) into s_pk / s_pv ----
  uint32_t jw = chunk_first[vb];  // the Gaussian (depth index) that holds position cs
  uint32_t done = 0;
  while (done < ce) {  // workgroup-uniform; each window covers at least kFuseWindow - 1 positions
    for (int q = tid; q < TILE; q += kSortThreads) s_owner[q] = 0u;
    __syncthreads();
    const uint64_t lo = cs + done, hi = cs + ce;
    {
      const uint64_t j = (uint64_t)jw + (uint32_t)tid;
      const uint4 d = j < (uint64_t)n ? drec[j] : make_uint4(0xFFFFFFFFu, 0u, 1u, 0u);
      s_off[tid] = d.x;
      s_tb[tid] = d.y;
      s_w[tid] = d.z;
      s_g[tid] = d.w;
      if (!targs.tight) {
        if (d.x >= lo && d.x < hi) atomicMax(&s_owner[d.x - lo], (uint32_t)tid);
      } else if (d.x < hi) {
        // tight rows: the Gaussian's positions run row by row, each row a run of tile ids. The
        // run holding position a >= lo leaves at chunk position a - cs its tile id (s_pk), its
        // Gaussian (s_pv) and the marker a - cs + 1, which the max-scan hands to the run.
        const uint4 r = targs.rec[d.w];  // (count, first tile, width, height)
        const TightShape ts = tight_of(targs, d.w);  // its loads in flight with rec's
        if ((uint64_t)d.x + r.x > lo) {
          const int x0 = (int)(d.y % (uint32_t)tiles_x), y0 = (int)(d.y / (uint32_t)tiles_x);
          uint64_t pos = d.x;
          for (uint32_t y = 0; y < r.w && pos < hi; ++y) {
            const int2 sp = tight_row(ts, y0 + (int)y, x0, x0 + (int)r.z);
            const uint32_t len = (uint32_t)(sp.y - sp.x);
            if (len > 0 && pos + len > lo) {
              const uint64_t a = pos > lo ? pos : lo;
              const uint32_t pc = (uint32_t)(a - cs);
              s_pk[pc] = (uint32_t)(y0 + (int)y) * (uint32_t)tiles_x + (uint32_t)sp.x + (uint32_t)(a - pos);
              s_pv[pc] = d.w;
              s_owner[pc - done] = pc + 1u;
            }
            pos += len;
          }
        }
      }
    }
    __syncthreads();
    // positions below the last window Gaussian's start are covered by this window
    const uint32_t last_off = s_off[kFuseWindow - 1];
    const uint64_t cover = (uint64_t)jw + kFuseWindow - 1 < (uint64_t)n && (uint64_t)last_off < hi
                               ? (uint64_t)last_off : hi;
    const uint32_t lim = (uint32_t)(cover - cs);
    // inclusive max-scan of the markers: owner of each position
    uint32_t o[kEmitPer];
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < kEmitPer; ++q) {
      o[q] = max(run, s_owner[tid * kEmitPer + q]);
      run = o[q];
    }
    uint32_t mx;
    const uint32_t before = block_scan1024<uint32_t>(run, 0u, s_wsum, &mx,
                                                      [](uint32_t x, uint32_t y) { return max(x, y); });
#pragma unroll
    for (int q = 0; q < kEmitPer; ++q) s_owner[tid * kEmitPer + q] = max(before, o[q]);
    __syncthreads();
    if (!targs.tight) {
#pragma unroll
      for (int q = 0; q < kEmitPer; ++q) {
        const uint32_t p = done + (uint32_t)(q * kSortThreads + tid);
        if (p < lim) {
          const uint32_t li = s_owner[p - done];
          const uint32_t local = (uint32_t)(cs + p - s_off[li]);
          const uint32_t ww = s_w[li];
          const uint32_t row = local / ww, col = local - row * ww;
          s_pk[p] = s_tb[li] + row * (uint32_t)tiles_x + col;
          s_pv[p] = s_g[li];
        }
      }
    } else {
      // every position of [lo, cover) has a run start at or below it (the run holding lo starts
      // there); read all first, the run starts are overwritten with their own values after
      uint32_t tk[kEmitPer], tv[kEmitPer];
#pragma unroll
      for (int q = 0; q < kEmitPer; ++q) {
        const uint32_t p = done + (uint32_t)(q * kSortThreads + tid);
        tk[q] = tv[q] = 0u;
        if (p < lim) {
          const uint32_t st = s_owner[p - done] - 1u;
          tk[q] = s_pk[st] + (p - st);
          tv[q] = s_pv[st];
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kEmitPer; ++q) {
        const uint32_t p = done + (uint32_t)(q * kSortThreads + tid);
        if (p < lim) {
          s_pk[p] = tk[q];
          s_pv[p] = tv[q];
        }
      }
    }
    __syncthreads();
    // the next window starts at the Gaussian holding position lim (the window's last one)
    if (lim < ce) jw += kFuseWindow - 1;
    done = lim;
  }

  // ---- the first pass over the tile's pairs ----
  uint32_t k[ITEMS], v[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint32_t idx = (uint32_t)(wave * 64 * ITEMS + i * 64 + lane);
    k[i] = idx < ce ? s_pk[idx] : 0u;
    v[i] = idx < ce ? s_pv[idx] : 0u;
  }
  __syncthreads();  // s_mem now takes the per-wave digit counts
  for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) s_mem[i] = 0u;
  const uint32_t h = tid < kRadix ? hist[tid] : 0u;
  __syncthreads();
  radix_tile<FINAL, ITEMS>(k, v, (uint32_t)P, (uint32_t)cs, vb, shift, bits, h, s_mem, s_dpre, s_goff, s_wsum,
                           status, keys_out, vals_out, out_keys64, depth_bits);
}

// ---------------------------------------------------------------------------------------------
// Small frames (N <= kSmallMaxN): the depth order from sorted blocks and merge ranks, two launches
// instead of the key-computing pass, four radix passes and the scan.
//   k_small_local  workgroup b < nb sorts block b (ids [4096 b, 4096 b + 4096)) by depth key in
//                  LDS (radix passes of up to 9 bits over the bits the block's keys span) and
//                  writes the sorted keys, ids and the exclusive prefix of their tile counts; it
//                  also adds its Gaussians' rectangle rows into its own row of per-tile count
//                  differences (tmat); the other workgroups only clear the control block and
//                  look-back words
//   k_small_merge  kSmallSplit workgroups per block, 1024 keys each: every key's place in the depth
//                  order is its place in its block plus, for every other block, how many of that
//                  block's keys come first (binary search over all N keys held in LDS; an earlier
//                  block's equal keys have smaller ids and come first); its first pair position is
//                  the sum of the matching tile-count prefixes. It writes the depth-ordered
//                  records and the emission chunks' first Gaussians as the scan does. Its last
//                  workgroup is the tile finalizer: it sums the blocks' count rows and writes the
//                  ranges, the pair-sort histograms, P and the raster plan.
// The order is the stable (depth bits, id) order of the radix path, bit for bit.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallBlock = kSortTile;  // 4096 Gaussians per block, four per thread
constexpr int kSmallMaxBlocks = 9;
constexpr int32_t kSmallMaxN = kSmallBlock * kSmallMaxBlocks;  // every key in 144 KB of LDS
constexpr uint32_t kSmallMaxTiles = 16383;                      // the difference array in LDS
constexpr int kLocalBits = 9;
constexpr int kLocalRadix = 1 << kLocalBits;
constexpr int kMergeThreads = kSortThreads;                     // the finalizer's workgroup size
constexpr int kMergeItems = 1;
constexpr int kSmallSplit = kSmallBlock / (kMergeThreads * kMergeItems);  // merge workgroups per block
// k_small_local's dynamic LDS (words): per-wave digit counts, keys, values, tile counts by local
// index, then the block's difference array
constexpr uint32_t kLocalCnt = kSortWaves * kLocalRadix;
constexpr uint32_t kLocalSortWords = kLocalCnt + 3 * kSmallBlock;
constexpr uint32_t kCountFixedWords = kFinStep + kFinAuxWords;  // the finalizer's LDS

struct SmallArgs {
  int32_t n;
  uint32_t nb;          // blocks
  const float* depths;
  const uint32_t* tiles;
  const float* means2d;
  const int32_t* radii;
  int32_t tiles_x, tiles_y;
  uint4* rec;           // [n] (count, first tile, width, height) in id order
  uint32_t* skey;       // [nb, 4096] block-sorted depth keys (0xFFFFFFFF: not drawn)
  uint32_t* sid;        // [nb, 4096] their ids
  uint32_t* cpre;       // [nb, 4096] exclusive prefix of their tile counts in block-sorted order
  uint32_t* btot;       // [nb] block totals of the tile counts
  uint32_t* tmat;       // [nb, tmat_stride] per-block difference arrays of the per-tile counts
  uint32_t tmat_stride;
  uint32_t* zero_a;     // cleared: the control block up to its pair-sort histograms
  size_t zero_a_words;
  uint32_t* zero_b;     // cleared: the pair look-back words
  size_t zero_b_words;
};

// Exclusive sum over the values of the first `nwaves` waves (the others pass 0), with DPP wave
// scans; two barriers. s_wsum holds at least nwaves words.
__device__ __forceinline__ uint32_t block_excl_scan_dpp(uint32_t v, int nwaves, uint32_t* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_incl_scan_dpp(v);
  if (wave < nwaves && lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave && w < nwaves; ++w) before += s_wsum[w];
  __syncthreads();
  return before + inc - v;
}

// One stable radix pass over `bits` (<= 9) bits at `shift` of the workgroup's 4096 items, in LDS:
// item i of lane l of wave w is element 256 w + 64 i + l on entry; the pass leaves the sequence
// in s_k / s_v in its new order and, unless `last`, reloads the items from there.
__device__ __forceinline__ void local_radix_pass(uint32_t (&k)[kSortItems], uint32_t (&v)[kSortItems], int shift,
                                                 int bits, bool last, uint32_t* s_cnt, uint32_t* s_k,
                                                 uint32_t* s_v, uint32_t* s_dig, uint32_t* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t radix = 1u << bits, mask = radix - 1u;
  // the first 2^bits counters of every wave (each wave clears its own)
  for (uint32_t i = lane; i < radix; i += 64) s_cnt[wave * kLocalRadix + i] = 0u;
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t rank[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t d = (k[i] >> shift) & mask;
    // all kLocalBits ballots, unconditionally: the digit's bits above `bits` are 0 in every lane
    // and leave the match mask unchanged
    const uint64_t m = match_digit<kLocalBits>(d, kLocalBits, ~0ull);
    const uint32_t r = (uint32_t)__popcll(m & lt_mask);
    const uint32_t pre = s_cnt[wave * kLocalRadix + d];
    rank[i] = pre + r;
    asm volatile("" : "+v"(rank[i]));
    if (r == 0) s_cnt[wave * kLocalRadix + d] = pre + (uint32_t)__popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per digit (threads below 2^bits): the waves' exclusive offsets and the digit total, the 16
  // counters loaded together; then the digit totals' exclusive scan
  uint32_t tot = 0;
  if ((uint32_t)tid < radix) {
    uint32_t c[kSortWaves];
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) c[w] = s_cnt[w * kLocalRadix + tid];
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      s_cnt[w * kLocalRadix + tid] = tot;
      tot += c[w];
    }
  }
  const uint32_t dex = block_excl_scan_dpp((uint32_t)tid < radix ? tot : 0u, kLocalRadix / 64, s_wsum);
  if ((uint32_t)tid < radix) s_dig[tid] = dex;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t d = (k[i] >> shift) & mask;
    const uint32_t pos = s_dig[d] + s_cnt[wave * kLocalRadix + d] + rank[i];
    s_k[pos] = k[i];
    s_v[pos] = v[i];
  }
  __syncthreads();
  if (!last) {
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
      const uint32_t e = (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
      k[i] = s_k[e];
      v[i] = s_v[e];
    }
  }
}

__global__ __launch_bounds__(kSortThreads) void k_small_local(SmallArgs sa, TileCountArgs ta) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_dig[kLocalRadix];
  __shared__ uint32_t s_wsum[kSortWaves];
  __shared__ uint32_t s_mm[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x >= sa.nb) {  // workgroup-uniform: clearing only
    const size_t base_w = (size_t)(blockIdx.x - sa.nb) * kSortThreads + tid;
    const size_t gsz = (size_t)(gridDim.x - sa.nb) * kSortThreads;
    for (size_t i = base_w; i < sa.zero_a_words; i += gsz) sa.zero_a[i] = 0u;
    for (size_t i = base_w; i < sa.zero_b_words; i += gsz) sa.zero_b[i] = 0u;
    return;
  }
  uint32_t* s_cnt = s_dyn;
  uint32_t* s_k = s_cnt + kLocalCnt;
  uint32_t* s_v = s_k + kSmallBlock;
  uint32_t* s_tc = s_v + kSmallBlock;
  uint32_t* s_diff = s_tc + kSmallBlock;
  const uint32_t b = blockIdx.x;
  const uint32_t base = b * (uint32_t)kSmallBlock;
  const uint32_t len = (uint32_t)sa.n - base < (uint32_t)kSmallBlock ? (uint32_t)sa.n - base : (uint32_t)kSmallBlock;
  for (uint32_t t = tid; t <= ta.ntiles; t += kSortThreads) s_diff[t] = 0u;
  if (tid == 0) {
    s_mm[0] = 0xFFFFFFFFu;
    s_mm[1] = 0u;
  }
  // element e = 256 w + 64 i + l of the block (id base + e)
  uint32_t key[kSortItems], tc[kSortItems];
  uint4 rc[kSortItems];
  float2 m[kSortItems];
  int2 r[kSortItems];
  float z[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {  // all loads in flight before any is used
    const uint32_t e = (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    const bool valid = e < len;
    const uint32_t g = base + e;
    tc[i] = valid ? sa.tiles[g] : 0u;
    z[i] = valid ? sa.depths[g] : 0.0f;
    m[i] = valid ? *reinterpret_cast<const float2*>(sa.means2d + 2 * (size_t)g) : make_float2(0.0f, 0.0f);
    r[i] = valid ? *reinterpret_cast<const int2*>(sa.radii + 2 * (size_t)g) : make_int2(0, 0);
  }
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    key[i] = tc[i] > 0 ? __float_as_uint(z[i]) : 0xFFFFFFFFu;
    uint32_t tb = 0, w = 1, h = 0;
    if (tc[i] > 0) {
      const TileRect rt = tile_rect(m[i].x, m[i].y, (float)r[i].x, (float)r[i].y, sa.tiles_x, sa.tiles_y);
      tb = (uint32_t)(rt.y0 * sa.tiles_x + rt.x0);
      w = (uint32_t)(rt.x1 - rt.x0);
      h = (uint32_t)(rt.y1 - rt.y0);
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
    rc[i] = make_uint4(tc[i], tb, w, h);
    if (e < len) sa.rec[base + e] = rc[i];
    s_tc[e] = tc[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
  }
  __syncthreads();  // s_mm and s_diff initialised
  if (lane == 0) {
    atomicMin(&s_mm[0], kmin);
    atomicMax(&s_mm[1], kmax);
  }
  // the block's pairs per tile: rows of its rectangles into its difference array
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
    tile_rows_item(ta, rc[i], base + e, e < len, s_diff);
  }
  __syncthreads();
  // codes: drawn keys minus the block's smallest, every other element one past the largest, so
  // that they sort last in element order; only the bits the codes span are sorted
  uint32_t lo = s_mm[0], hi = s_mm[1];
  if (lo > hi) lo = hi = 0u;  // nothing drawn in this block
  const uint32_t vmax = hi - lo + 1u;
  const int tbits = 32 - __clz((int)vmax);
  uint32_t code[kSortItems], val[kSortItems];
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    code[i] = key[i] != 0xFFFFFFFFu ? key[i] - lo : vmax;
    val[i] = (uint32_t)(wave * 64 * kSortItems + i * 64 + lane);
  }
  for (int sh = 0; sh < tbits; sh += kLocalBits) {  // workgroup-uniform
    const int bits = tbits - sh < kLocalBits ? tbits - sh : kLocalBits;
    local_radix_pass(code, val, sh, bits, sh + kLocalBits >= tbits, s_cnt, s_k, s_v, s_dig, s_wsum);
  }
  // the block's row of the difference array
  for (uint32_t t = tid; t <= ta.ntiles; t += kSortThreads) sa.tmat[(size_t)b * sa.tmat_stride + t] = s_diff[t];
  // sorted order, four consecutive elements per thread: raw keys, ids, tile-count prefix
  uint32_t ok[kSortItems], oid[kSortItems], oc[kSortItems];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < kSortItems; ++i) {
    const uint32_t e = (uint32_t)(tid * kSortItems + i);
    const uint32_t c = s_k[e], lv = s_v[e];
    ok[i] = c == vmax ? 0xFFFFFFFFu : c + lo;
    oid[i] = base + lv;
    oc[i] = s_tc[lv];
    own += oc[i];
  }
  const uint32_t run = block_excl_scan_dpp(own, kSortWaves, s_wsum);
  uint4 pre;
  pre.x = run;
  pre.y = pre.x + oc[0];
  pre.z = pre.y + oc[1];
  pre.w = pre.z + oc[2];
  const size_t o4 = (size_t)b * (kSmallBlock / 4) + tid;
  reinterpret_cast<uint4*>(sa.skey)[o4] = make_uint4(ok[0], ok[1], ok[2], ok[3]);
  reinterpret_cast<uint4*>(sa.sid)[o4] = make_uint4(oid[0], oid[1], oid[2], oid[3]);
  reinterpret_cast<uint4*>(sa.cpre)[o4] = pre;
  if (tid == kSortThreads - 1) sa.btot[b] = pre.w + oc[3];
}

// Merge ranks: workgroup kSmallSplit b + s takes block b's sorted elements [1024 s, 1024 s + 1024),
// one per thread; workgroup kSmallSplit nb is the tile-count finalizer. Dynamic LDS: max(nb 4096,
// the finalizer's) words (every block's sorted keys).
__global__ __launch_bounds__(kMergeThreads) void k_small_merge(SmallArgs sa, uint4* __restrict__ drec,
                                                               uint32_t* __restrict__ chunk_first, uint64_t capacity,
                                                               Ctrl* ctrl, int64_t* __restrict__ user_num_pairs,
                                                               uint32_t lds_words, TileCountArgs ta) {
  extern __shared__ uint32_t s_dyn[];
  const int tid = threadIdx.x;
  const uint32_t nb = sa.nb;
  if (blockIdx.x == nb * kSmallSplit) {  // workgroup-uniform: the tile-count finalizer
    tile_finalize(ta, s_dyn, lds_words);
    return;
  }
  const uint32_t b = blockIdx.x / kSmallSplit, sub = blockIdx.x % kSmallSplit;
  {  // every block's sorted keys into LDS, eight 16-byte loads in flight per thread
    const uint32_t nq = nb * (kSmallBlock / 4);
    const uint4* src = reinterpret_cast<const uint4*>(sa.skey);
    uint4* dst = reinterpret_cast<uint4*>(s_dyn);
    for (uint32_t q0 = 0; q0 < nq; q0 += 8 * kMergeThreads) {
      uint4 t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t q = q0 + (uint32_t)(j * kMergeThreads + tid);
        t[j] = q < nq ? src[q] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t q = q0 + (uint32_t)(j * kMergeThreads + tid);
        if (q < nq) dst[q] = t[j];
      }
    }
  }
  if (blockIdx.x == 0 && tid == 0) {  // P: the sum of the block totals
    uint64_t P = 0;
    for (uint32_t j = 0; j < nb; ++j) P += sa.btot[j];
    ctrl->num_pairs = P;
    ctrl->eff_pairs = P <= capacity ? P : 0u;
    if (user_num_pairs) *user_num_pairs = (int64_t)P;
  }
  __syncthreads();
  auto block_len = [&](uint32_t bb) {
    const uint32_t rest = (uint32_t)sa.n - bb * (uint32_t)kSmallBlock;
    return rest < (uint32_t)kSmallBlock ? rest : (uint32_t)kSmallBlock;
  };
  const uint32_t len_b = block_len(b);
  const uint32_t e0 = sub * (uint32_t)(kMergeThreads * kMergeItems) + (uint32_t)tid * kMergeItems;
  // for each other block, how many of its keys come first: <= key for an earlier block (its equal
  // keys have smaller ids), < key for a later one. All searches advance together.
  uint32_t key[kMergeItems];
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) key[i] = s_dyn[b * kSmallBlock + e0 + (uint32_t)i];
  uint32_t pos[kSmallMaxBlocks][kMergeItems];
#pragma unroll
  for (int b2 = 0; b2 < kSmallMaxBlocks; ++b2)
#pragma unroll
    for (int i = 0; i < kMergeItems; ++i) pos[b2][i] = 0u;
  // branch-free: every step reads one key per (block, item), the index clamped into the block (a
  // block that is this one or does not exist has length 0 and reads block 0's first key), so all
  // reads of a step are in flight together
  uint32_t len2[kSmallMaxBlocks], kbase[kSmallMaxBlocks];
  bool before[kSmallMaxBlocks];
#pragma unroll
  for (int b2 = 0; b2 < kSmallMaxBlocks; ++b2) {
    const bool use = (uint32_t)b2 < nb && (uint32_t)b2 != b;
    len2[b2] = use ? block_len((uint32_t)b2) : 0u;
    kbase[b2] = use ? (uint32_t)b2 * kSmallBlock : 0u;
    before[b2] = (uint32_t)b2 < b;
  }
#pragma unroll
  for (uint32_t step = kSmallBlock; step > 0; step >>= 1) {
#pragma unroll
    for (int b2 = 0; b2 < kSmallMaxBlocks; ++b2) {
#pragma unroll
      for (int i = 0; i < kMergeItems; ++i) {
        const uint32_t p = pos[b2][i] + step;
        const uint32_t idx = kbase[b2] + (p <= len2[b2] ? p - 1u : 0u);
        const uint32_t x = s_dyn[idx];
        const bool first = before[b2] ? x <= key[i] : x < key[i];
        pos[b2][i] = (p <= len2[b2] && first) ? p : pos[b2][i];
      }
    }
  }
  // ranks and first pair positions: every block's prefix loads issued together
  uint32_t rank[kMergeItems], g[kMergeItems];
  uint64_t off[kMergeItems];
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) {
    const uint32_t e = e0 + (uint32_t)i;
    rank[i] = e;
    off[i] = e < len_b ? sa.cpre[(size_t)b * kSmallBlock + e] : 0u;
    g[i] = e < len_b ? sa.sid[(size_t)b * kSmallBlock + e] : 0u;
  }
#pragma unroll
  for (int b2 = 0; b2 < kSmallMaxBlocks; ++b2) {
    if (len2[b2] == 0u) continue;  // uniform
#pragma unroll
    for (int i = 0; i < kMergeItems; ++i) {
      const uint32_t p = pos[b2][i];
      rank[i] += p;
      off[i] += p < len2[b2] ? sa.cpre[(size_t)b2 * kSmallBlock + p] : sa.btot[b2];
    }
  }
  uint4 r[kMergeItems];
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) r[i] = sa.rec[g[i]];  // g = 0 past the block: a valid index, unused
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) {
    const uint32_t e = e0 + (uint32_t)i;
    if (e >= len_b) break;
    drec[rank[i]] = make_uint4(off[i] < 0xFFFFFFFFull ? (uint32_t)off[i] : 0xFFFFFFFFu, r[i].y, r[i].z, g[i]);
    const uint64_t end = off[i] + r[i].x;
    for (uint64_t c = (off[i] + kEmitChunk - 1) / kEmitChunk * kEmitChunk; c < end && c < capacity; c += kEmitChunk)
      chunk_first[c / kEmitChunk] = rank[i];
  }
}

// The raster plan of a frame without pairs: natural tile order, no extra work items or checkpoints.
__global__ void k_empty_plan(uint32_t* __restrict__ plan, uint32_t ntiles) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    plan[kPlanChunk] = kPlanMinChunk;
    plan[kPlanExtra] = 0;
    plan[kPlanCheckpoints] = 0;
    plan[kPlanSplit] = 0;
  }
  if (i < ntiles) {
    plan[kPlanOrder + i] = i;
    plan[kPlanOrder + ntiles + i] = 0;
  }
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t count, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------------------------
// workspace layout: [ctrl | scan look-back | depth look-back | pair look-back] are zeroed by
// k_bin_prep; the rest is written before it is read
// ---------------------------------------------------------------------------------------------
// [ctrl | pair look-back] is what the small-frame path zeroes, [ctrl .. zero_end) what the radix
// path zeroes
struct BinLayout {
  size_t ctrl, pstatus, small_zero_end, scan_status, dstatus, tdiff, zero_end;
  size_t dhist, dkA, dvA, dkB, dvB, rec, drec, chunk_first, pkB, pvB;
  size_t skey, sid, cpre, btot, tmat, total;
  uint32_t nbN, nbS, nbCap, nbEmit, nbSmall, tmat_stride;
  bool small;
  int tile_bits, npass, pshift[3], pbits[3];
};

BinLayout bin_layout(int32_t n, int64_t cap, const gs_camera* cam) {
  BinLayout L{};
  const size_t A = 256;
  const int64_t ntiles = (int64_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  int tb = 1;
  while (((int64_t)1 << tb) < ntiles) ++tb;
  L.tile_bits = tb;
  L.npass = (tb + 7) / 8;
  // the tile-id bits split evenly over the passes (14 = 7 + 7, not 8 + 6): fewer digits per pass
  // mean fewer look-back columns
  for (int p = 0, sh = 0; p < L.npass; ++p) {
    L.pbits[p] = tb / L.npass + (p < tb % L.npass ? 1 : 0);
    L.pshift[p] = sh;
    sh += L.pbits[p];
  }
  L.nbN = (uint32_t)((n + kSortTile - 1) / kSortTile);
  L.nbS = (uint32_t)((n + kScanTile - 1) / kScanTile);
  L.nbCap = (uint32_t)((cap + kSortTile - 1) / kSortTile);
  L.nbEmit = (uint32_t)((cap + kEmitChunk - 1) / kEmitChunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, A);
    return at;
  };
  // small frames: every key in one workgroup's LDS, a block's difference array in LDS
  L.small = n <= kSmallMaxN && ntiles <= (int64_t)kSmallMaxTiles;
  L.nbSmall = L.small ? (uint32_t)((n + kSmallBlock - 1) / kSmallBlock) : 0u;
  L.tmat_stride = (uint32_t)align_up((size_t)ntiles + 1, 64);
  L.ctrl = take(sizeof(Ctrl));
  L.pstatus = take((size_t)L.npass * L.nbCap * kRadix * 4);
  L.small_zero_end = off;
  L.scan_status = take((size_t)L.nbS * 8);
  L.dstatus = take((size_t)4 * L.nbN * kRadix * 4);
  L.tdiff = take(((size_t)ntiles + 1) * 4);
  L.zero_end = off;
  L.dhist = take((size_t)L.nbN * 4 * kRadix * 4);
  L.dkA = take((size_t)n * 4);
  L.dvA = take((size_t)n * 4);
  L.dkB = take((size_t)n * 4);
  L.dvB = take((size_t)n * 4);
  L.rec = take((size_t)n * 16);
  L.drec = take((size_t)n * 16);
  L.chunk_first = take((size_t)L.nbEmit * 4);
  L.pkB = take((size_t)cap * 4);
  L.pvB = take((size_t)cap * 4);
  L.skey = take((size_t)L.nbSmall * kSmallBlock * 4);
  L.sid = take((size_t)L.nbSmall * kSmallBlock * 4);
  L.cpre = take((size_t)L.nbSmall * kSmallBlock * 4);
  L.btot = take((size_t)L.nbSmall * 4);
  L.tmat = take((size_t)L.nbSmall * L.tmat_stride * 4);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_raster_plan_words(const gs_camera* cam) {
  if (!cam || cam->width <= 0 || cam->height <= 0) return 0;
  const size_t ntiles = (size_t)((cam->width + 15) / 16) * ((cam->height + 15) / 16);
  return plan_words(ntiles);
}

extern "C" size_t gs_bin_workspace_bytes(int32_t n, int64_t pair_capacity, const gs_camera* cam) {
  if (n < 0 || pair_capacity < 0 || !cam || cam->width <= 0 || cam->height <= 0) return 0;
  return bin_layout(n, pair_capacity, cam).total;
}

namespace {
// The small-frame kernels take up to 112 and 144 KB of dynamic LDS: raise their limits (64 KB by default)
// once per device.
constexpr size_t kSmallLocalLds = (size_t)(kLocalSortWords + kSmallMaxTiles + 1) * 4;
constexpr size_t kSmallMergeLds = (size_t)kSmallMaxBlocks * kSmallBlock * 4;
static_assert(kSmallLocalLds + 4 * (kLocalRadix + kSortWaves + 2) <= 160 * 1024, "LDS of a compute unit");
static_assert((size_t)kCountFixedWords * 4 <= kSmallMergeLds && kSmallMergeLds + 8 <= 160 * 1024,
              "LDS of a compute unit");
std::mutex g_lds_mu;
bool g_lds_set[64] = {};
gs_status raise_small_lds_limits() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return set_error(GS_ERR_DEVICE, "gs_bin_and_sort: no current device");
  std::lock_guard<std::mutex> lock(g_lds_mu);
  if (g_lds_set[dev]) return GS_OK;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_small_local), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kSmallLocalLds) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(k_small_merge), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kSmallMergeLds) != hipSuccess)
    return check_launch("gs_bin_and_sort: raising the LDS limit");
  g_lds_set[dev] = true;
  return GS_OK;
}

gs_status bin_and_sort(int32_t n, const gs_projected* proj, const gs_camera* cam, void* d_workspace,
                       size_t workspace_bytes, int64_t pair_capacity, uint64_t* d_keys, uint32_t* d_ids,
                       uint32_t* d_tile_ranges, uint32_t* d_raster_plan, int64_t* d_num_pairs, int64_t* h_num_pairs,
                       void* stream) {
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
  if (n > 0 && cam->tight_tiles && (!proj->d_conics || !proj->d_opacities))
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort: tight_tiles needs the conics and opacities");
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
    if (d_raster_plan)
      hipLaunchKernelGGL(k_empty_plan, dim3((unsigned)((ntiles + 255) / 256)), dim3(256), 0, s, d_raster_plan,
                         (uint32_t)ntiles);
    return check_launch("gs_bin_and_sort");
  }
  char* ws = (char*)d_workspace;
  Ctrl* ctrl = (Ctrl*)(ws + L.ctrl);
  uint32_t *dkA = (uint32_t*)(ws + L.dkA), *dvA = (uint32_t*)(ws + L.dvA), *dkB = (uint32_t*)(ws + L.dkB),
           *dvB = (uint32_t*)(ws + L.dvB), *dhist = (uint32_t*)(ws + L.dhist);
  uint64_t* scan_status = (uint64_t*)(ws + L.scan_status);
  uint32_t* dstatus = (uint32_t*)(ws + L.dstatus);
  uint32_t* pstatus = (uint32_t*)(ws + L.pstatus);
  const int32_t tiles_x = (cam->width + 15) / 16, tiles_y = (cam->height + 15) / 16;
  // the tile-count arguments: extra workgroups count the pairs of every tile and finalize them
  TileCountArgs targs;
  targs.rec = (const uint4*)(ws + L.rec);
  targs.means2d = proj->d_means2d;
  targs.conics = proj->d_conics;
  targs.opac = proj->d_opacities;
  targs.tight = cam->tight_tiles;
  targs.n = n;
  targs.tiles_x = tiles_x;
  targs.ntiles = (uint32_t)ntiles;
  targs.tdiff = (uint32_t*)(ws + L.tdiff);
  targs.ranges = d_tile_ranges;
  targs.plan = d_raster_plan;
  targs.capacity = (uint64_t)pair_capacity;
  targs.npass = L.npass;
  for (int p = 0; p < 3; ++p) {
    targs.pshift[p] = p < L.npass ? L.pshift[p] : 0;
    targs.pbits[p] = p < L.npass ? L.pbits[p] : 0;
  }
  targs.hist_pair = &ctrl->hist_pair[0][0];
  targs.tmat = nullptr;
  targs.tmat_rows = 0;
  targs.tmat_stride = 0;
  targs.all_ranges = 0;
  // ping-pong of the pair sort: A = d_keys viewed as two u32 arrays of pair_capacity, B = workspace.
  // The last pass writes the 64-bit keys over A, so it reads B: pass p writes B when
  // npass - 2 - p is even, A otherwise.
  uint32_t* kA = (uint32_t*)d_keys;
  uint32_t* vA = kA ? kA + pair_capacity : nullptr;
  uint32_t *kB = (uint32_t*)(ws + L.pkB), *vB = (uint32_t*)(ws + L.pvB);
  if (L.small) {
    SmallArgs sa;
    sa.n = n;
    sa.nb = L.nbSmall;
    sa.depths = proj->d_depths;
    sa.tiles = proj->d_tiles_touched;
    sa.means2d = proj->d_means2d;
    sa.radii = proj->d_radii;
    sa.tiles_x = tiles_x;
    sa.tiles_y = tiles_y;
    sa.rec = (uint4*)(ws + L.rec);
    sa.skey = (uint32_t*)(ws + L.skey);
    sa.sid = (uint32_t*)(ws + L.sid);
    sa.cpre = (uint32_t*)(ws + L.cpre);
    sa.btot = (uint32_t*)(ws + L.btot);
    sa.tmat = (uint32_t*)(ws + L.tmat);
    sa.tmat_stride = L.tmat_stride;
    // cleared by the extra workgroups: the control block up to its pair-sort histograms (the
    // finalizer writes those in the same launch) and the pair look-back words
    sa.zero_a = (uint32_t*)(ws + L.ctrl);
    sa.zero_a_words = offsetof(Ctrl, hist_pair) / 4;
    sa.zero_b = pstatus;
    sa.zero_b_words = (L.small_zero_end - L.pstatus) / 4;
    const size_t zwords = sa.zero_a_words + sa.zero_b_words;
    const unsigned zblocks = (unsigned)std::min<size_t>((zwords + 16 * kSortThreads - 1) / (16 * kSortThreads), 256);
    const size_t lds_local = ((size_t)kLocalSortWords + ntiles + 1) * 4;
    const uint32_t merge_words = std::max<uint32_t>(L.nbSmall * kSmallBlock, kCountFixedWords);
    const size_t lds_merge = (size_t)merge_words * 4;
    const gs_status lst = raise_small_lds_limits();
    if (lst != GS_OK) return lst;
    {
      TimedScope ts("small_local", s);
      hipLaunchKernelGGL(k_small_local, dim3(L.nbSmall + zblocks), dim3(kSortThreads), lds_local, s, sa, targs);
    }
    targs.tmat = sa.tmat;
    targs.tmat_rows = L.nbSmall;
    targs.tmat_stride = L.tmat_stride;
    targs.all_ranges = 1;
    {
      TimedScope ts("small_merge", s);
      hipLaunchKernelGGL(k_small_merge, dim3(L.nbSmall * kSmallSplit + 1), dim3(kMergeThreads), lds_merge, s, sa,
                         (uint4*)(ws + L.drec), (uint32_t*)(ws + L.chunk_first), (uint64_t)pair_capacity, ctrl,
                         d_num_pairs, merge_words, targs);
    }
  } else {
  const size_t zero_words = (L.zero_end - L.ctrl) / 4;
  {
    // enough workgroups for the depth keys, and for zeroing about 32 words per thread
    const size_t zwords = zero_words + (size_t)(2 * ntiles);
    const size_t zblocks = (zwords + 32 * kSortThreads - 1) / (32 * kSortThreads);
    const unsigned blocks = (unsigned)std::max<size_t>(L.nbN, std::min<size_t>(zblocks, 2048));
    TimedScope ts("bin_prep", s);
    hipLaunchKernelGGL(k_bin_prep, dim3(blocks), dim3(kSortThreads), 0, s, n, proj->d_depths, proj->d_tiles_touched,
                       proj->d_means2d, proj->d_radii, tiles_x, tiles_y, (uint4*)(ws + L.rec), dkA, dvA, dhist,
                       L.nbN, (uint32_t*)(ws + L.ctrl), zero_words, d_tile_ranges, (size_t)(2 * ntiles));
  }
  // up to kDirectHistRows prep workgroups, each depth pass sums the per-workgroup histograms itself
  // (one launch fewer); beyond, every pass workgroup would re-read too many rows, and
  // k_hist_reduce sums them once
  const bool direct_hist = L.nbN <= (uint32_t)kDirectHistRows;
  if (!direct_hist) {
    TimedScope ts("hist_reduce", s);
    hipLaunchKernelGGL(k_hist_reduce, dim3(4, (L.nbN + kReduceRows - 1) / kReduceRows), dim3(kRadix), 0, s, dhist,
                       L.nbN, ctrl);
  }
  // pass 0 carries the tile-row workgroups, pass 1 the tile-count finalizer
  const uint32_t n_rows = (uint32_t)((n + kRowGaussians - 1) / kRowGaussians);
  for (int p = 0; p < 4; ++p) {
    const bool even = (p % 2) == 0;
    const uint32_t* hist = direct_hist ? dhist + p * kRadix : ctrl->hist_depth[p];
    const uint32_t n_extra = p == 0 ? n_rows : (p == 1 ? 1u : 0u);
    auto kern = p == 0 ? k_onesweep<false, 1, 4> : (p == 1 ? k_onesweep<false, 2, 4> : k_onesweep<false, 0, 4>);
    TimedScope ts("depth_sort_pass", s);
    // pass 0 sorts all n keys and drops the culled ones; the later passes sort the drawn ones
    hipLaunchKernelGGL(kern, dim3(L.nbN + n_extra), dim3(kSortThreads), 0, s, even ? dkA : dkB, even ? dvA : dvB,
                       even ? dkB : dkA, even ? dvB : dvA, (uint64_t*)nullptr, (const uint32_t*)nullptr,
                       (uint32_t)n, p == 0 ? (const uint64_t*)nullptr : &ctrl->n_visible, 8 * p, 8, hist,
                       direct_hist ? (int)L.nbN : 1, 4 * kRadix, dstatus + (size_t)p * L.nbN * kRadix,
                       &ctrl->tickets[p], n_extra, targs, p == 0 ? &ctrl->n_visible : (uint64_t*)nullptr);
  }
  {
    TimedScope ts("scan", s);
    hipLaunchKernelGGL(k_scan, dim3(L.nbS), dim3(kEmitThreads), 0, s, n, &ctrl->n_visible, dvA,
                       (const uint4*)(ws + L.rec), (uint4*)(ws + L.drec), (uint32_t*)(ws + L.chunk_first),
                       (uint64_t)pair_capacity, scan_status, ctrl, d_num_pairs);
  }
  }
  if (L.nbCap > 0) {
    auto out_A = [&](int p) { return ((L.npass - 2 - p) % 2) != 0; };
    {
      // emission and the first pass, one workgroup per 4096 pair positions
      TimedScope ts("emit_sort", s);
      const bool last = L.npass == 1;
      auto kern = last ? k_emit_sort<true> : k_emit_sort<false>;
      const bool oa = out_A(0);
      // large frames: the depth-ordered records of the drawn Gaussians only
      hipLaunchKernelGGL(kern, dim3(L.nbCap), dim3(kSortThreads), 0, s, &ctrl->eff_pairs, n,
                         L.small ? (const uint64_t*)nullptr : &ctrl->n_visible, (const uint4*)(ws + L.drec), (const uint32_t*)(ws + L.chunk_first), tiles_x, L.pshift[0],
                         L.pbits[0], ctrl->hist_pair[0], pstatus, &ctrl->tickets[4],
                         last ? (uint32_t*)nullptr : (oa ? kA : kB), last ? d_ids : (oa ? vA : vB),
                         last ? d_keys : (uint64_t*)nullptr,
                         last ? (const uint32_t*)proj->d_depths : (const uint32_t*)nullptr, targs);
    }
    // 8 keys per lane (8192 per workgroup) for large pair buffers
    const bool wide = pair_capacity > ((int64_t)1 << 19);
    const unsigned grid = wide ? (L.nbCap + 1) / 2 : L.nbCap;
    for (int p = 1; p < L.npass; ++p) {
      const int shift = L.pshift[p], bits = L.pbits[p];
      const bool last = p == L.npass - 1;
      const bool in_A = out_A(p - 1);
      uint32_t *ki = in_A ? kA : kB, *vi = in_A ? vA : vB;
      uint32_t *ko = in_A ? kB : kA, *vo = in_A ? vB : vA;
      auto kern = last ? (wide ? k_onesweep<true, 0, 8> : k_onesweep<true, 0, 4>)
                       : (wide ? k_onesweep<false, 0, 8> : k_onesweep<false, 0, 4>);
      TimedScope ts("pair_sort_pass", s);
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kSortThreads), 0, s, ki, vi, last ? (uint32_t*)nullptr : ko,
                         last ? d_ids : vo, last ? d_keys : (uint64_t*)nullptr,
                         last ? (const uint32_t*)proj->d_depths : (const uint32_t*)nullptr, 0u, &ctrl->eff_pairs,
                         shift, bits, ctrl->hist_pair[p], 1, 0, pstatus + (size_t)p * L.nbCap * kRadix,
                         &ctrl->tickets[4 + p], 0u, targs, (uint64_t*)nullptr);
    }
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
}  // namespace

extern "C" gs_status gs_bin_and_sort(int32_t n, const gs_projected* proj, const gs_camera* cam, void* d_workspace,
                                     size_t workspace_bytes, int64_t pair_capacity, uint64_t* d_keys,
                                     uint32_t* d_ids, uint32_t* d_tile_ranges, uint32_t* d_raster_plan,
                                     int64_t* d_num_pairs, int64_t* h_num_pairs, void* stream) {
  return bin_and_sort(n, proj, cam, d_workspace, workspace_bytes, pair_capacity, d_keys, d_ids, d_tile_ranges,
                      d_raster_plan, d_num_pairs, h_num_pairs, stream);
}

// ---------------------------------------------------------------------------------------------
// The binning without allocation: its workspace is this file-scope device array, one copy per
// GPU, held until the process ends. Host code never passes the array's name to a kernel (on the
// host it only names a shadow); it passes the device address hipGetSymbolAddress returns, taken
// once per device with that device current.
// ---------------------------------------------------------------------------------------------
namespace {
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

gs_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(GS_ERR_DEVICE, "gs_bin_and_sort_noalloc: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(GS_ERR_DEVICE, std::string("gs_bin_and_sort_noalloc: hipGetSymbolAddress: ") +
                                          hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GS_OK;
}
}  // namespace

extern "C" size_t gs_bin_noalloc_max_workspace_bytes(void) { return kStaticScratchBytes; }

extern "C" gs_status gs_bin_and_sort_noalloc(int32_t n, const gs_projected* proj, const gs_camera* cam,
                                             int64_t pair_capacity, uint64_t* d_keys, uint32_t* d_ids,
                                             uint32_t* d_tile_ranges, uint32_t* d_raster_plan,
                                             int64_t* d_num_pairs, void* stream) {
  if (n < 0 || pair_capacity < 0 || !cam || cam->width <= 0 || cam->height <= 0)
    return set_error(GS_ERR_INVALID_ARG, "gs_bin_and_sort_noalloc: n < 0, capacity < 0 or an invalid camera");
  const size_t need = bin_layout(n, pair_capacity, cam).total;
  if (need > kStaticScratchBytes)
    return set_error(GS_ERR_LIMIT, "gs_bin_and_sort_noalloc: this frame needs " + std::to_string(need) +
                                       " bytes of workspace, above the static maximum of " +
                                       std::to_string(kStaticScratchBytes) + " (use gs_bin_and_sort)");
  void* ws = nullptr;
  const gs_status st = scratch_of_current_device(&ws);
  if (st != GS_OK) return st;
  return bin_and_sort(n, proj, cam, ws, kStaticScratchBytes, pair_capacity, d_keys, d_ids, d_tile_ranges,
                      d_raster_plan, d_num_pairs, nullptr, stream);
}
