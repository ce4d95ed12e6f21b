/*
 * gs.h -- C ABI of the MI355X (gfx950) tile-based 3D Gaussian Splatting rasterizer.
 *
 * Method: "Gaussian splatting in PyTorch" (coderigor.dev/lessons/py-gaussian-splatting), whose
 * sections 1-6 define what is computed: raw parameters and their activations (section 1),
 * Sigma = R S S^T R^T (section 2), the world->camera transform and EWA projection with the
 * widened-frustum clamp (section 3), the eps2d dilation, conic and radius (section 4), the
 * front-to-back blend with early termination (section 5) and the backward (section 6). The tile
 * pipeline -- project, count, emit, sort, range, blend -- is the one of "SplatRs: The Week the
 * Gap Closed" (section "Throughput: the tile rasterizer"); the backward walks each tile back to
 * front and recovers the transmittance by division (section 6 of the PyTorch lesson).
 *
 * Conventions shared by every entry point:
 *  - Pointers named d_* are device pointers (HBM of the current HIP device), h_* host pointers.
 *    Arrays are contiguous, row-major, fp32 unless typed otherwise. The caller allocates and owns
 *    every buffer; the library never frees or retains a caller pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls enqueue work on
 *    it and return without waiting, except gs_bin_and_sort when asked for the pair count on the
 *    host (h_num_pairs != NULL), which waits once for it.
 *  - Every call returns a gs_status; on anything but GS_OK, gs_last_error() describes it and no
 *    output has been written past what the status documents. No exception crosses the ABI.
 *  - Calls with disjoint buffers may run concurrently on different streams.
 *  - Image layout: pixel (i, j) is row i, column j and is sampled at (j + 0.5, i + 0.5);
 *    images are [height, width, 3]; tiles are 16 x 16 pixels, tile id = ty * tiles_x + tx with
 *    tiles_x = ceil(width / 16), tiles_y = ceil(height / 16).
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_TILE_SIZE 16
#define GS_MAX_SH_DEGREE 3

typedef enum gs_status {
  GS_OK = 0,
  GS_ERR_INVALID_ARG = 1, /* bad size, NULL pointer, degree, or a non-finite camera */
  GS_ERR_CAPACITY = 2,    /* the pair buffers are too small: *h_num_pairs holds the need */
  GS_ERR_LIMIT = 3,       /* a size beyond what the kernels index (n or capacity >= 2^30, tiles > 2^24) */
  GS_ERR_DEVICE = 4       /* a HIP runtime error; gs_last_error() has its text */
} gs_status;

/* Pinhole camera with OpenCV axes (+x right, +y down, +z forward): section 3 of the PyTorch
 * lesson takes a world->camera viewmat [4,4] and intrinsics K. Read on the host only. */
typedef struct gs_camera {
  float viewmat[16];   /* row-major [R | t; 0 0 0 1], world -> camera */
  float fx, fy, cx, cy; /* intrinsics in pixels (cx = width/2 centres the image) */
  int32_t width, height;
  float near_plane;    /* Gaussians with camera z <= near_plane are culled (0.01 typical) */
  float background[3]; /* composited with the final transmittance */
  /* Variants of section 4 of the PyTorch lesson (0 = the default; set them to 0 otherwise):
   * radius_mode 0: gsplat's opacity-aware per-axis extent; 1: the original 3DGS radius
   *   ceil(3 sqrt(lambda_max)) (root argument floored at 0.1) on both axes. A splat then draws
   *   only in the tiles of its rectangle, even where its alpha would still reach 1/255.
   * antialiased 1: the blend's opacity is o sqrt(det Sigma2d / det(Sigma2d + 0.3 I)), Sigma2d
   *   the projected covariance before the dilation (gsplat's "antialiased" mode, Mip-Splatting's
   *   2D filter); the cull and the extent use that opacity, and the backward differentiates it.
   * tight_tiles 1: a splat is listed only in the tiles of its rectangle whose pixel-centre box
   *   its ellipse sigma <= s2 reaches, s2 = k^2 / 2 (k the opacity-aware extent, at most 3.33)
   *   widened by 0.002 + s (0.002 + q / 65536), q = A C / (A C - B^2) of the conic: section 4's
   *   tighter bound, fewer pairs for the sort and the blend, the same image (every pixel with
   *   alpha >= 1/255 stays listed). Decided row by row of the rectangle in fp32; tiles_touched
   *   is then the tight count (0: not drawn).
   * The same options must be given to every call of one iteration. */
  int32_t radius_mode;
  int32_t antialiased;
  int32_t tight_tiles;
} gs_camera;

/* Projected records, structure of arrays of length n, written by gs_project. A Gaussian is
 * drawn iff tiles_touched > 0 (then radii > 0). Undefined projections (camera z <= near, or a
 * non-finite input or derived value) are all zeros; defined but undrawn ones (opacity < 1/255,
 * or no tile on screen) keep their projected values with radii = (0, 0), tiles_touched = 0. */
typedef struct gs_projected {
  float* d_means2d;          /* [n,2] pixel coordinates of the mean (not clamped) */
  float* d_conics;           /* [n,3] (A, B, C) = inverse of the dilated 2D covariance */
  float* d_depths;           /* [n]   camera-space z */
  float* d_opacities;        /* [n]   sigmoid(logit) */
  float* d_colors;           /* [n,3] sum_lm k_lm B_lm(view direction); degree 0: the RGB */
  int32_t* d_radii;          /* [n,2] ceil(k sqrt(Sigma'_xx)), ceil(k sqrt(Sigma'_yy)) */
  uint32_t* d_tiles_touched; /* [n]   tiles of the tile rectangle */
} gs_projected;

/*
 * gs_project -- activations, covariance, EWA projection, culling, conic, radius, tile count and
 * colour for every Gaussian (sections 1-4 of the PyTorch lesson).
 *   q = quat / max(|quat|, 1e-12) (w, x, y, z); s = exp(log_scale); o = 1 / (1 + exp(-logit));
 *   Sigma = M M^T, M = R(q) diag(s); t = W mean + w0; Sigma_c = W Sigma W^T;
 *   J = [[fx/z, 0, -fx x~/z^2], [0, fy/z, -fy y~/z^2]] with x~/z, y~/z clamped to the view
 *   widened by 0.3 tan(half FoV) per side; Sigma' = J Sigma_c J^T + 0.3 I = [[a, b], [b, c]];
 *   conic = (c, -b, a) / max(ac - b^2, 1e-10); mean2d = (fx x/z + cx, fy y/z + cy);
 *   k = min(3.33, sqrt(2 ln(255 o))), radii = ceil(k sqrt(a)), ceil(k sqrt(c)) (opacity-aware
 *   extent: alpha < 1/255 outside it); tile rectangle [floor((mean2d - r)/16),
 *   ceil((mean2d + r)/16)) clamped to the grid; colour from real SH of degree sh_degree, scaled
 *   so that the degree-0 basis is 1, at the unit direction from the camera centre to the mean.
 *   exp and log are evaluated with a fixed written-out fp32 algorithm (Cody-Waite exp, atanh-
 *   series log), so radii, rectangles and tile counts are reproducible bit for bit.
 * Inputs (device, fp32): d_means [n,3], d_log_scales [n,3], d_quats [n,4] (w,x,y,z, any norm),
 *   d_opacity_logits [n], d_sh [n, (sh_degree+1)^2, 3] coefficient-major.
 * Output: every array of *out, length n.
 * Errors: GS_ERR_INVALID_ARG for n < 0, a NULL pointer with n > 0, sh_degree outside 0..3,
 *   width/height <= 0, fx/fy <= 0 or a non-finite camera field.
 */
gs_status gs_project(int32_t n, int32_t sh_degree, const float* d_means, const float* d_log_scales,
                     const float* d_quats, const float* d_opacity_logits, const float* d_sh,
                     const gs_camera* cam, const gs_projected* out, void* stream);

/*
 * gs_bin_and_sort -- count, emit, sort and range ("project, count, emit, sort, range" of the
 * SplatRs tile rasterizer). For every drawn Gaussian i and every tile (tx, ty) of its rectangle
 * (with cam->tight_tiles, every tile of the rectangle its ellipse reaches, row by row) it forms
 * the key (ty * tiles_x + tx) << 32 | float_bits(depth_i) and the value i, sorts the
 * pairs by key, keeping equal keys in ascending i (stable), and writes per tile the range
 * [start, end) of its pairs in the sorted list ((0, 0) for an empty tile).
 * Implementation: the Gaussians put in stable depth order (up to 36,864 of them and 16,383 tiles:
 * blocks of 4096 sorted in LDS and merge-ranked against each other; beyond: a stable LSD radix
 * sort), the first pair position of each from a prefix of the tile counts in depth order,
 * emission of (tile, i) pairs in that order, and a stable LSD radix sort of the pairs by tile
 * id (Onesweep-style single-pass passes with decoupled look-back).
 * Inputs: n and proj (from gs_project with the same camera; it reads depths, tiles_touched,
 *   means2d and radii, and with tight_tiles also conics and opacities); d_workspace of at least
 *   gs_bin_workspace_bytes(n, pair_capacity, cam) bytes (device, 256-byte aligned, contents
 *   arbitrary on entry and need not persist between calls); pair_capacity = length of d_keys
 *   and d_ids.
 * Outputs: d_keys [P] uint64, d_ids [P] uint32, d_tile_ranges [tiles, 2] uint32;
 *   d_raster_plan (optional, gs_raster_plan_words(cam) uint32): how the raster calls schedule the
 *   frame -- the tiles in an order that gives each of the GPU's 8 XCDs (workgroup b runs on XCD
 *   b mod 8) its own list of tiles, 2x1 blocks of neighbouring tiles together, each list with the
 *   tiles holding more pairs first (by the bit length of the count, empty tiles last), the lists
 *   interleaved; a chunk length L (a power of two >= 128 with P <= 4096 L),
 *   and for every tile of two or more chunks of L list entries its checkpoint slots and the
 *   backward's extra work items (its chunks after the first); P itself goes to
 *   *d_num_pairs (device int64, optional, written on `stream`) and to *h_num_pairs (host,
 *   optional). d_keys doubles as scratch during the call.
 * Waiting: with h_num_pairs == NULL nothing waits: the call only enqueues kernels, sized by the
 *   capacity, that stop at the device-side count. With h_num_pairs != NULL it waits once on
 *   `stream` to read P and returns GS_ERR_CAPACITY when P > pair_capacity.
 * Capacity overflow (P > pair_capacity): every tile range is (0, 0), so a later blend draws the
 *   background only; the first pair_capacity entries of d_keys/d_ids hold unspecified values and
 *   nothing past them is written; P is still reported in full. Callers that do not wait check
 *   *d_num_pairs <= pair_capacity later.
 * Errors: GS_ERR_INVALID_ARG (as gs_project, or a workspace below the size needed, or a
 *   misaligned d_workspace / d_keys / d_num_pairs), GS_ERR_LIMIT (n or pair_capacity >= 2^30,
 *   or more than 2^24 tiles).
 */
size_t gs_bin_workspace_bytes(int32_t n, int64_t pair_capacity, const gs_camera* cam);
size_t gs_raster_plan_words(const gs_camera* cam);
gs_status gs_bin_and_sort(int32_t n, const gs_projected* proj, const gs_camera* cam, void* d_workspace,
                          size_t workspace_bytes, int64_t pair_capacity, uint64_t* d_keys, uint32_t* d_ids,
                          uint32_t* d_tile_ranges, uint32_t* d_raster_plan, int64_t* d_num_pairs,
                          int64_t* h_num_pairs, void* stream);

/*
 * gs_bin_and_sort_noalloc -- gs_bin_and_sort for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and results,
 * with no workspace argument and no host wait. Its workspace is a static device array of
 * gs_bin_noalloc_max_workspace_bytes() bytes (64 MiB), one per GPU, allocated with the library's
 * code and held until the process ends; the call allocates nothing and calls no allocating
 * routine. Every call on one GPU shares that array, so calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be serialized by the caller; the
 * kernels clear what must start at zero, so one call's leftovers do not reach the next.
 * Arguments: as gs_bin_and_sort without d_workspace, workspace_bytes and h_num_pairs; P goes to
 *   *d_num_pairs (device int64, optional). Results are those of gs_bin_and_sort (overflow
 *   included: every range (0, 0) and P reported in full).
 * Errors: those of gs_bin_and_sort, and GS_ERR_LIMIT when gs_bin_workspace_bytes(n,
 *   pair_capacity, cam) exceeds the static maximum (nothing is enqueued; use gs_bin_and_sort),
 *   GS_ERR_DEVICE when the array's device address cannot be taken.
 */
size_t gs_bin_noalloc_max_workspace_bytes(void);
gs_status gs_bin_and_sort_noalloc(int32_t n, const gs_projected* proj, const gs_camera* cam, int64_t pair_capacity,
                                  uint64_t* d_keys, uint32_t* d_ids, uint32_t* d_tile_ranges,
                                  uint32_t* d_raster_plan, int64_t* d_num_pairs, void* stream);

/*
 * gs_rasterize_fwd -- per-pixel front-to-back alpha blending over the pixel's tile list (section
 * 5 of the PyTorch lesson): for each pair in the tile's range, in order,
 *   sigma = 0.5 (A dx^2 + C dy^2) + B dx dy with (dx, dy) = mean2d - pixel centre;
 *   alpha = min(0.99, o exp(-sigma)); skip if sigma < 0 or alpha < 1/255;
 *   stop before adding when T (1 - alpha) <= 1e-4; else pixel += colour alpha T, T *= 1 - alpha;
 * and finally pixel += T background.
 * Inputs: proj, d_ids and d_tile_ranges from gs_bin_and_sort for the same camera;
 *   d_raster_plan (optional, NULL = tiles in id order) from that gs_bin_and_sort call: the tiles
 *   are taken in its order (scheduling only, the results do not change); d_raster_ws (optional,
 *   gs_raster_workspace_bytes() bytes, device, zero-filled by the caller before its first use,
 *   used only with a plan; every call leaves its synchronisation words zero again): the forward
 *   stores there, for tiles longer than the plan's chunk length L, per chunk of L list entries
 *   and per pixel the transmittance after the chunk and the colour the chunk added, which lets
 *   gs_rasterize_bwd split such tiles. With it, a tile of more than 512 entries and three or more
 *   chunks of 2 L entries is blended chunk by chunk in parallel: a chunk starts from the product
 *   of the earlier chunks' transmittance factors (1 - alpha multiplied over their contributing
 *   splats), and the image is summed chunk by chunk, so results equal those without a workspace
 *   up to rounding.
 *   Calls that share a workspace must not overlap (one stream, or ordered streams).
 * Outputs: d_image [h,w,3]; d_depth [h,w] (optional, NULL = not rendered): the depth channel,
 *   the splats' camera z through the same weights, D = sum z_i alpha_i T_i with background depth
 *   0 (section 5: any channel, depth included, blends with the same weights; with a workspace
 *   its per-chunk parts are stored too, for a backward with d_dL_ddepth);
 *   d_final_T [h,w] the transmittance after the last added splat;
 *   d_n_contrib [h,w] uint32: number of tile-list entries up to and including the last added
 *   splat (0 if none). d_eval_count: NULL, or a device uint64 to which the number of
 *   (pixel, entry) evaluations is added (a work counter for measurement).
 * Deterministic: no atomics on the outputs; each pixel is written once.
 * Any per-Gaussian three-channel quantity blends with the same weights (section 5: any channel
 * goes through the blend): pass it as proj->d_colors with a camera background of 0; given to
 * gs_rasterize_bwd as degree-0 coefficients (basis 1) it comes back as their gradient.
 */
size_t gs_raster_workspace_bytes(void);
gs_status gs_rasterize_fwd(int32_t n, const gs_projected* proj, const gs_camera* cam, const uint32_t* d_ids,
                           const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan, void* d_raster_ws,
                           float* d_image, float* d_depth, float* d_final_T, uint32_t* d_n_contrib,
                           uint64_t* d_eval_count, void* stream);

/*
 * gs_rasterize_fwd_l1 -- gs_rasterize_fwd with the L1 term of the training loss (section 7 of
 * the PyTorch lesson) fused into the blend: as each pixel's colour is finished, its gradient
 * dL/dimage = sign(image - target) / (3 h w) (sign(0) = 0) is written beside it, bit for bit what
 * gs_loss_l1 writes from the same image, without reading the image back.
 * Inputs and outputs: those of gs_rasterize_fwd, plus d_target [h,w,3] (device) and
 * d_dL_dimage [h,w,3] (device, written for every pixel). The loss value itself is not formed
 * (gs_loss_l1 gives it). Errors: those of gs_rasterize_fwd; GS_ERR_INVALID_ARG for a NULL
 * d_target or d_dL_dimage.
 */
gs_status gs_rasterize_fwd_l1(int32_t n, const gs_projected* proj, const gs_camera* cam, const uint32_t* d_ids,
                              const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan, void* d_raster_ws,
                              float* d_image, float* d_depth, float* d_final_T, uint32_t* d_n_contrib,
                              const float* d_target, float* d_dL_dimage, uint64_t* d_eval_count, void* stream);

/*
 * gs_rasterize_bwd -- gradients of a loss L with respect to the raw parameters, given
 * dL/dimage (section 6 of the PyTorch lesson). Each tile is walked back to front from each
 * pixel's last contributor; T_i = T_{i+1} / (1 - alpha_i) is recovered by division (the 0.99
 * cap keeps 1 - alpha >= 0.01) and the blend weights are recomputed, never stored:
 *   dC/dc_i = alpha_i T_i,  dC/dalpha_i = c_i T_i - S_i / (1 - alpha_i),
 *   S_i = sum_{j>i} c_j alpha_j T_j + T_final background,
 * then through alpha = o exp(-sigma) (no gradient where the 0.99 cap is active) to the 2D mean,
 * conic and opacity, and by the chain rule of gs_project to the raw parameters. Culled
 * Gaussians get exactly zero; radii, rectangles, keys and the sort carry no gradient.
 * Inputs: the raw parameters and camera given to gs_project, its proj, the d_ids/d_tile_ranges
 *   of gs_bin_and_sort, d_final_T/d_n_contrib of gs_rasterize_fwd, d_dL_dimage [h,w,3];
 *   d_raster_plan and d_raster_ws (optional): with both -- the plan and workspace the forward was
 *   given -- each work item of the plan (one chunk of L list entries of a tile) runs as its own
 *   workgroup, an inner chunk starting from the forward's checkpoints (the transmittance after
 *   the chunk, and S = T_final background + the colour each later chunk added); with a plan
 *   only, the tiles are taken in its order; without, in id order;
 *   d_dL_ddepth [h,w] (optional, NULL = none): the gradient on the depth channel of
 *   gs_rasterize_fwd, which then joins the colour channels (dD/dz_i = alpha_i T_i and a depth
 *   term in dD/dalpha_i) and reaches the means through the camera z; with d_raster_ws the
 *   forward must have rendered d_depth into that workspace;
 *   d_workspace of at least gs_bwd_workspace_bytes(n) bytes (device).
 * Outputs (overwritten, not accumulated): d_grad_means [n,3], d_grad_log_scales [n,3],
 *   d_grad_quats [n,4], d_grad_opacity_logits [n], d_grad_sh [n,(sh_degree+1)^2,3], and
 *   d_grad_means2d [n,2] (may be NULL) = dL/d mean2d. d_eval_count as in gs_rasterize_fwd.
 * Per-Gaussian sums use fp32 atomics, so results may differ in the last bits run to run.
 */
size_t gs_bwd_workspace_bytes(int32_t n);
gs_status gs_rasterize_bwd(int32_t n, int32_t sh_degree, const float* d_means, const float* d_log_scales,
                           const float* d_quats, const float* d_opacity_logits, const float* d_sh,
                           const gs_camera* cam, const gs_projected* proj, const uint32_t* d_ids,
                           const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan, const void* d_raster_ws,
                           const float* d_final_T, const uint32_t* d_n_contrib, const float* d_dL_dimage,
                           const float* d_dL_ddepth, void* d_workspace, size_t workspace_bytes,
                           float* d_grad_means, float* d_grad_log_scales, float* d_grad_quats,
                           float* d_grad_opacity_logits, float* d_grad_sh, float* d_grad_means2d,
                           uint64_t* d_eval_count, void* stream);

/*
 * gs_rasterize_bwd_deterministic -- gs_rasterize_bwd with bitwise-reproducible gradients: the
 * same inputs give the same bits on every run. No floating-point atomics: the 2D gradient of
 * each (tile, Gaussian) pair is written to its own slot -- a Gaussian's pairs are contiguous
 * from the prefix sum of tiles_touched in id order, row-major over its tile rectangle (with
 * tight_tiles, over each row's tight run) -- and the slots of a Gaussian are added in an order
 * fixed by its pair count alone: a Gaussian of at most 16 pairs by one lane in slot order, a
 * larger one by a whole wave (lane l adds slots l, l + 64, ... in order, then a fixed lane
 * tree); inside a tile the four waves' sums of a splat are added in wave order.
 * Arguments as gs_rasterize_bwd, plus pair_capacity: at least the P of gs_bin_and_sort (the
 *   capacity given to it will do); d_dL_ddepth as in gs_rasterize_bwd; d_workspace (256-byte aligned) of at least
 *   gs_bwd_det_workspace_bytes(n, pair_capacity) bytes. If P > pair_capacity every gradient is 0
 *   (as after a binning overflow). Results agree with gs_rasterize_bwd to rounding.
 * Errors: those of gs_rasterize_bwd, GS_ERR_INVALID_ARG for pair_capacity < 0 or a misaligned
 *   workspace, GS_ERR_LIMIT for pair_capacity >= 2^30.
 */
size_t gs_bwd_det_workspace_bytes(int32_t n, int64_t pair_capacity);
gs_status gs_rasterize_bwd_deterministic(int32_t n, int32_t sh_degree, const float* d_means,
                                         const float* d_log_scales, const float* d_quats,
                                         const float* d_opacity_logits, const float* d_sh, const gs_camera* cam,
                                         const gs_projected* proj, const uint32_t* d_ids,
                                         const uint32_t* d_tile_ranges, const uint32_t* d_raster_plan,
                                         const void* d_raster_ws, const float* d_final_T,
                                         const uint32_t* d_n_contrib, const float* d_dL_dimage,
                                         const float* d_dL_ddepth, int64_t pair_capacity, void* d_workspace,
                                         size_t workspace_bytes,
                                         float* d_grad_means, float* d_grad_log_scales, float* d_grad_quats,
                                         float* d_grad_opacity_logits, float* d_grad_sh, float* d_grad_means2d,
                                         uint64_t* d_eval_count, void* stream);

/*
 * gs_loss_l1 -- the L1 photometric term of the training loss (section 7 of the PyTorch lesson:
 * (1 - lambda) L1 + lambda (1 - SSIM)): L = mean |image - target| over h*w*3 values, so
 * dL/dimage = sign(image - target) / (3 h w) with sign(0) = 0.
 * Inputs: d_image, d_target [h,w,3]. Outputs: d_dL_dimage [h,w,3]; d_loss (device float[1],
 * may be NULL) receives L. Arrays must be 4-byte aligned (16-byte aligned ones take a float4
 * path). Errors: GS_ERR_INVALID_ARG for a size <= 0, a NULL array or a misaligned one.
 */
gs_status gs_loss_l1(int32_t width, int32_t height, const float* d_image, const float* d_target,
                     float* d_dL_dimage, float* d_loss, void* stream);

/*
 * gs_loss_l1_ssim -- the full training loss of section 7 of the PyTorch lesson,
 * L = (1 - lambda) L1 + lambda (1 - SSIM) (lambda = 0.2 there), and dL/dimage. SSIM is that of
 * Wang, Bovik, Sheikh and Simoncelli (2004), which the lesson names without fixing a window: per
 * channel, local means and (co)variances under an 11 x 11 Gaussian window of standard deviation
 * 1.5 (normalised to sum 1) over the image padded with zeros, C1 = 0.01^2, C2 = 0.03^2,
 * S = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy + C2)), and SSIM the
 * mean of S over the h*w*3 values; L1 = mean |image - target| with sign(0) = 0 in its gradient.
 * Inputs: d_image, d_target [h,w,3]; lambda in [0, 1]; d_workspace (device, 256-byte aligned) of
 * at least gs_loss_ssim_workspace_bytes(width, height) bytes, contents arbitrary on entry.
 * Outputs: d_dL_dimage [h,w,3]; d_loss (device float[1], may be NULL) receives L, its sums added
 * in a fixed order (the same bits every run).
 * Errors: GS_ERR_INVALID_ARG for a size <= 0, a NULL pointer, lambda outside [0, 1], a small or
 * misaligned workspace; GS_ERR_LIMIT for 9 h w >= 2^31.
 */
size_t gs_loss_ssim_workspace_bytes(int32_t width, int32_t height);
gs_status gs_loss_l1_ssim(int32_t width, int32_t height, const float* d_image, const float* d_target, float lambda,
                          void* d_workspace, size_t workspace_bytes, float* d_dL_dimage, float* d_loss,
                          void* stream);

/*
 * gs_adam_step -- one optimizer step on the raw parameters: Adam (Kingma and Ba 2015, in the form
 * torch.optim.Adam uses, which the fitting loop of section 7 of the PyTorch lesson calls) with a
 * learning rate per group (the lesson lists per-parameter rates for 3DGS training), plus the
 * splat-size penalty of the distillation write-up ("The backward pass I deleted": a loss term on
 * splat size; its form there is unstated and read here as size_penalty * mean over Gaussians of
 * sum_j exp(l_j), which adds size_penalty * exp(l_j) / n to dL/dl_j before the update).
 * Per value: m <- b1 m + (1 - b1) g, v <- b2 v + (1 - b2) g^2,
 *            p <- p - lr / (1 - b1^step) * m / (sqrt(v) / sqrt(1 - b2^step) + eps).
 * Inputs: n, sh_degree and the raw parameter arrays as in gs_project (updated in place), the
 *   gradients of gs_rasterize_bwd (same layouts), step >= 1 (the count of steps so far, this one
 *   included), cfg (host). SH band 0 (the first 3 values of each Gaussian's [K,3] block) takes
 *   lr_sh_dc, the other bands lr_sh_rest.
 * State: d_m, d_v (device, gs_adam_state_floats(n, sh_degree) floats each, zero before step 1,
 *   owned by the caller and carried between steps), laid out as means [n,3], log_scales [n,3],
 *   quats [n,4], opacity_logits [n], sh [n,K,3] in that order, each group starting at a float
 *   offset that is a multiple of 64 (the previous groups' sizes, each rounded up to 64 floats).
 *   Groups whose arrays are 16-byte aligned and hold a multiple of 4 values take a float4 path.
 * Errors: GS_ERR_INVALID_ARG (n < 0, sh_degree outside 0..3, step < 1, a NULL pointer with
 *   n > 0, a negative or non-finite rate or penalty, a beta outside [0, 1), eps <= 0),
 *   GS_ERR_LIMIT (3 K n >= 2^31).
 */
typedef struct {
  float lr_means, lr_log_scales, lr_quats, lr_opacity, lr_sh_dc, lr_sh_rest;
  float beta1, beta2, eps;
  float size_penalty;
} gs_adam_config;
size_t gs_adam_state_floats(int32_t n, int32_t sh_degree);
gs_status gs_adam_step(int32_t n, int32_t sh_degree, int32_t step, const gs_adam_config* cfg, float* d_means,
                       float* d_log_scales, float* d_quats, float* d_opacity_logits, float* d_sh,
                       const float* d_grad_means, const float* d_grad_log_scales, const float* d_grad_quats,
                       const float* d_grad_opacity_logits, const float* d_grad_sh, float* d_m, float* d_v,
                       void* stream);

/* Human-readable name of a status, and a thread-local description of the last non-OK return. */
const char* gs_status_string(gs_status s);
const char* gs_last_error(void);

/*
 * Kernel timing for measurement. While enabled, every kernel the library launches is bracketed
 * by HIP events on its stream. gs_timing_collect waits for those events and returns up to `max`
 * (name, milliseconds) records in launch order, then forgets them; it returns the number of
 * records written. Not thread-safe; intended for a single measuring thread.
 */
gs_status gs_timing_enable(int32_t on);
int32_t gs_timing_collect(const char** names, float* ms, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
