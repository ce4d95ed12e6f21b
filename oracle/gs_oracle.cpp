// CPU oracle for the differentiable tile-based 3D Gaussian Splatting rasterizer.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path loads, links or calls this file: only
// tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may. It shares no code, header,
// table or constant generator with the HIP library; both follow the same published definitions.
//
// What it computes, and where each step is defined ("Gaussian splatting in PyTorch",
// coderigor.dev/lessons/py-gaussian-splatting, cited below as "the PyTorch lesson"):
//   * raw parameters -> activations (section 1), Sigma = R S S^T R^T (section 2),
//   * world -> camera, EWA Jacobian with the widened-frustum clamp, eps2d dilation (section 3),
//   * conic, opacity-aware per-axis radius and the tile rectangle (section 4),
//   * the per-pixel front-to-back blend with the 1/255 skip, the 0.99 cap and the T <= 1e-4
//     stop-before-add (section 5), per pixel: every pixel walks the un-culled Gaussians whose
//     tile rectangle holds its tile (the tiled renderer's lists; with the default opacity-aware
//     radius that is every Gaussian that can reach the pixel, i.e. the dense render) in one
//     stable global depth order (section 5's argsort(depths, stable=True)),
//   * the analytic backward of all of the above (section 6 names the chain; the formulas are
//     derived from the forward definitions and checked against central finite differences).
// Binning is brute force: enumerate each Gaussian's tile rectangle, std::stable_sort the
// (tile | depth) keys, scan for per-tile ranges ("SplatRs: The Week the Gap Closed", section
// "Throughput: the tile rasterizer": project, count, emit, sort, range, blend).
//
// Precision. Everything is templated on T. T = float is the kernel's precision: every decision
// that yields an integer (culling, radii, tile rectangles, the blend's skip/stop decisions) is
// taken in fp32, in the op order written here, with contraction off (-ffp-contract=off). The
// activations exp/log use "D1", a written-out Cody-Waite exp and an atanh-series log, so that
// both sides of a parity check can evaluate the same function bit for bit. Values (pixels,
// gradients) are accumulated in double from those fp32 decisions. T = double is used for the
// closed-form pins and the finite-difference gradient checks.
//
// Readings where the pages leave a step open:
//   - radius rule: gsplat's per-axis extent with the opacity-aware k = min(3.33, sqrt(2 ln(255 o)))
//     (section 4 of the PyTorch lesson); Gaussians with o < 1/255 are culled;
//   - tile rectangle [floor((mu - r)/16), ceil((mu + r)/16)) clamped to the grid;
//   - key = tile_id << 32 | float_bits(depth), tile_id = ty * tiles_x + tx, depth = camera z;
//   - ties in depth keep ascending Gaussian id (stable sort);
//   - pixel (i, j) is sampled at (j + 0.5, i + 0.5);
//   - termination T * (1 - alpha) <= 1e-4 stops without adding (gsplat's comparison);
//   - near plane: cull z <= near; any non-finite input or derived value culls;
//   - colour: real spherical harmonics scaled so that the degree-0 basis is 1 (no offset, no clamp).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ---------------------------------------------------------------------------------------------
// D1: deterministic fp32 exp and log.
// exp: Cody & Waite, "Software Manual for the Elementary Functions" (1980), additive range
// reduction x = k ln2 + r with ln2 split into a 14-bit head (k * head is exact for |k| <= 256)
// and a tail, then the degree-7 Taylor polynomial of e^r by Horner's rule with fused
// multiply-adds, and e^x = 2^k e^r. The input is clamped to [-87, 88] so the result is a normal.
// log: x = m 2^e with m in [sqrt(1/2), sqrt(2)), ln m = 2 atanh(s), s = (m - 1)/(m + 1), the odd
// series of atanh to s^9, then ln x = e ln2 + ln m.
// ---------------------------------------------------------------------------------------------
float d1_expf(float x) {
  if (x != x) return x;
  if (x < -87.0f) x = -87.0f;
  if (x > 88.0f) x = 88.0f;
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e4p-1f;
  const float ln2_lo = 0x1.7f7d1cp-20f;
  float k = std::rint(x * log2e);
  float r = (x - k * ln2_hi) - k * ln2_lo;
  float p = 0x1.a01a02p-13f;          // 1/7!
  p = std::fma(p, r, 0x1.6c16c2p-10f); // 1/6!
  p = std::fma(p, r, 0x1.111112p-7f);  // 1/5!
  p = std::fma(p, r, 0x1.555556p-5f);  // 1/4!
  p = std::fma(p, r, 0x1.555556p-3f);  // 1/3!
  p = std::fma(p, r, 0.5f);
  p = std::fma(p, r, 1.0f);
  p = std::fma(p, r, 1.0f);
  return std::ldexp(p, (int)k);
}

float d1_logf(float x) {
  if (x != x) return x;
  if (x < 0.0f) return NAN;
  if (x == 0.0f) return -INFINITY;
  if (x == INFINITY) return x;
  int e = 0;
  float m = std::frexp(x, &e);  // x = m 2^e, m in [0.5, 1)
  if (m < 0x1.6a09e6p-1f) {     // below sqrt(1/2): move to [sqrt(1/2), sqrt(2))
    m = m * 2.0f;
    e = e - 1;
  }
  float s = (m - 1.0f) / (m + 1.0f);
  float s2 = s * s;
  float q = 0x1.c71c72p-4f;         // 1/9
  q = std::fma(q, s2, 0x1.24924ap-3f); // 1/7
  q = std::fma(q, s2, 0x1.99999ap-3f); // 1/5
  q = std::fma(q, s2, 0x1.555556p-2f); // 1/3
  float t = s2 * q;
  float two_s = 2.0f * s;
  float lnm = std::fma(two_s, t, two_s);
  float fe = (float)e;
  float r = std::fma(fe, 0x1.7f7d1cp-20f, lnm);  // e * ln2_lo + ln m
  return std::fma(fe, 0x1.62e4p-1f, r);           // + e * ln2_hi (exact product)
}

template <class T> struct Act;
template <> struct Act<float> {
  static float exp(float x) { return d1_expf(x); }
  static float log(float x) { return d1_logf(x); }
};
template <> struct Act<double> {
  static double exp(double x) { return std::exp(x); }
  static double log(double x) { return std::log(x); }
};

template <class T> bool finite(T x) { return std::isfinite(x); }

// ---------------------------------------------------------------------------------------------
// Camera: row-major world->camera viewmat [4,4] with OpenCV axes (+x right, +y down, +z
// forward) and pinhole intrinsics (the PyTorch lesson, section 3). Packed as 27 numbers:
// viewmat[16], fx, fy, cx, cy, near, bg[3], radius_mode, antialiased, tight_tiles; width and
// height are passed separately. The first two options are the variants section 4 of the lesson lists:
// radius_mode 0 = gsplat's opacity-aware per-axis extent, 1 = the original 3DGS radius
// ceil(3 sqrt(lambda_max)) for both axes; antialiased 1 = opacity times the compensation
// sqrt(det Sigma2d / det(Sigma2d + 0.3 I)) (gsplat's "antialiased" mode, Mip-Splatting's 2D
// filter), read with Sigma2d the covariance before the eps2d dilation. tight_tiles 1 lists a
// Gaussian only in the tiles of its rectangle that its ellipse reaches (tight_span below): the
// tighter bound the lesson's section 4 says means fewer sort keys and less blending.
// ---------------------------------------------------------------------------------------------
constexpr int kNumCam = 27;
template <class T> struct Cam {
  T V[16];
  T fx, fy, cx, cy, near_plane;
  T bg[3];
  int W, H;
  int tiles_x, tiles_y;
  int radius_mode, antialiased, tight_tiles;
};

template <class T> Cam<T> make_cam(const T* p, int W, int H) {
  Cam<T> c;
  for (int i = 0; i < 16; ++i) c.V[i] = p[i];
  c.fx = p[16]; c.fy = p[17]; c.cx = p[18]; c.cy = p[19]; c.near_plane = p[20];
  c.bg[0] = p[21]; c.bg[1] = p[22]; c.bg[2] = p[23];
  c.radius_mode = (int)p[24];
  c.antialiased = (int)p[25];
  c.tight_tiles = (int)p[26];
  c.W = W; c.H = H;
  c.tiles_x = (W + 15) / 16;
  c.tiles_y = (H + 15) / 16;
  return c;
}

// ---------------------------------------------------------------------------------------------
// Real spherical harmonics, scaled by sqrt(4 pi) so that the degree-0 function is 1, order
// m = -l..l, no Condon-Shortley phase. d = (x, y, z) is a unit vector. The pages do not define
// view-dependent colour; this is the textbook basis (orthonormal up to the 4 pi scale).
// ---------------------------------------------------------------------------------------------
template <class T> void sh_basis(int degree, T x, T y, T z, T* B) {
  const T s3 = (T)std::sqrt(3.0), s15 = (T)std::sqrt(15.0), s5h = (T)(std::sqrt(5.0) / 2.0),
          s15h = (T)(std::sqrt(15.0) / 2.0), s358 = (T)std::sqrt(35.0 / 8.0),
          s105 = (T)std::sqrt(105.0), s218 = (T)std::sqrt(21.0 / 8.0), s7h = (T)(std::sqrt(7.0) / 2.0),
          s105h = (T)(std::sqrt(105.0) / 2.0);
  B[0] = (T)1;
  if (degree < 1) return;
  B[1] = s3 * y;
  B[2] = s3 * z;
  B[3] = s3 * x;
  if (degree < 2) return;
  B[4] = s15 * x * y;
  B[5] = s15 * y * z;
  B[6] = s5h * ((T)3 * z * z - (T)1);
  B[7] = s15 * x * z;
  B[8] = s15h * (x * x - y * y);
  if (degree < 3) return;
  B[9] = s358 * y * ((T)3 * x * x - y * y);
  B[10] = s105 * x * y * z;
  B[11] = s218 * y * ((T)5 * z * z - (T)1);
  B[12] = s7h * z * ((T)5 * z * z - (T)3);
  B[13] = s218 * x * ((T)5 * z * z - (T)1);
  B[14] = s105h * z * (x * x - y * y);
  B[15] = s358 * x * (x * x - (T)3 * y * y);
}

// Partial derivatives of each B_lm polynomial above with respect to (x, y, z), treated as free
// variables; callers project them onto the tangent plane of the sphere.
void sh_basis_grad(int degree, double x, double y, double z, double (*dB)[3]) {
  const double s3 = std::sqrt(3.0), s15 = std::sqrt(15.0), s5 = std::sqrt(5.0),
               s358 = std::sqrt(35.0 / 8.0), s105 = std::sqrt(105.0), s218 = std::sqrt(21.0 / 8.0),
               s7h = std::sqrt(7.0) / 2.0, s105h = std::sqrt(105.0) / 2.0;
  for (int k = 0; k < 16; ++k) dB[k][0] = dB[k][1] = dB[k][2] = 0.0;
  if (degree < 1) return;
  dB[1][1] = s3;
  dB[2][2] = s3;
  dB[3][0] = s3;
  if (degree < 2) return;
  dB[4][0] = s15 * y; dB[4][1] = s15 * x;
  dB[5][1] = s15 * z; dB[5][2] = s15 * y;
  dB[6][2] = 3.0 * s5 * z;
  dB[7][0] = s15 * z; dB[7][2] = s15 * x;
  dB[8][0] = s15 * x; dB[8][1] = -s15 * y;
  if (degree < 3) return;
  dB[9][0] = s358 * 6.0 * x * y; dB[9][1] = s358 * (3.0 * x * x - 3.0 * y * y);
  dB[10][0] = s105 * y * z; dB[10][1] = s105 * x * z; dB[10][2] = s105 * x * y;
  dB[11][1] = s218 * (5.0 * z * z - 1.0); dB[11][2] = s218 * 10.0 * y * z;
  dB[12][2] = s7h * (15.0 * z * z - 3.0);
  dB[13][0] = s218 * (5.0 * z * z - 1.0); dB[13][2] = s218 * 10.0 * x * z;
  dB[14][0] = s105h * 2.0 * x * z; dB[14][1] = -s105h * 2.0 * y * z; dB[14][2] = s105h * (x * x - y * y);
  dB[15][0] = s358 * (3.0 * x * x - 3.0 * y * y); dB[15][1] = -s358 * 6.0 * x * y;
}

// ---------------------------------------------------------------------------------------------
// Projection of one Gaussian, every intermediate kept for the backward.
// ---------------------------------------------------------------------------------------------
template <class T> struct Proj {
  bool defined;  // passed the near plane and every finiteness test: the float outputs are set
  bool culled;   // not drawn (undefined, o < 1/255, or no tile on screen): radii/tiles are 0
  // activations (section 1)
  T qn_raw, qn;      // |q| and max(|q|, 1e-12)
  T q[4];            // normalised (w, x, y, z)
  T s[3];            // exp(log_scale)
  T o;               // sigmoid(logit)
  // covariance (section 2)
  T R[9], M[9], Sig[9];
  // camera (section 3)
  T t[3], Sc[9];
  T xz, yz, jx, jy;  // x/z, y/z and the clamped J arguments z * clamp(.)
  bool clamp_x, clamp_y;
  T J[6];            // rows (J00 J01 J02), (J10 J11 J12)
  T a, b, c;         // dilated 2D covariance
  T a0, c0, det0;    // the diagonal and determinant before the dilation
  T comp;            // antialiased compensation sqrt(det0 / det) (1 when off)
  T o_eff;           // the opacity the blend uses: o comp
  T det_raw, det;
  T conic[3];
  T m2d[2];
  T k;               // opacity-aware extent in standard deviations
  T rx, ry;          // radii (already ceil'd and saturated)
  int rect[4];       // x0, y0, x1, y1 in tiles
  uint32_t tiles;
  T depth;
  T dir[3], dir_norm;  // unit view direction for SH and its length before normalising
  T color[3];
  int radius_3dgs;
};

// ---------------------------------------------------------------------------------------------
// Tight tile rows. A pixel centre q sees alpha >= 1/255 only where sigma(q - mu') <= ln(255 o),
// and never beyond sigma = k^2 / 2 with k = min(3.33, sqrt(2 ln(255 o))) (section 4's extent:
// past 3.33 sigma even o = 1 is below 1/255). Tile (tx, ty) of the rectangle is kept when the
// ellipse sigma <= s2 meets the box of its pixel centres [16 tx + 0.5, 16 tx + 15.5] x
// [16 ty + 0.5, 16 ty + 15.5]. s2 widens k^2 / 2 by 0.002 + s (0.002 + q / 65536) with
// q = A C / (A C - B^2) >= 1, the ratio that bounds the size of sigma's terms on the ellipse
// (4 s q), so that fp32 rounding of sigma or of the row bounds cannot drop a reached pixel.
// Per row (v = y - mu'_y over the row's centre rows clipped to |v| <= sqrt(2 s2 A / D)) the
// ellipse spans u = x - mu'_x in [L, R]; R is largest at v = -B t and L smallest at v = B t,
// t = sqrt(2 s2 / (C D)) (clamped into the row), with u = (-B v +- sqrt(2 s2 A - D v^2)) / A.
// The row keeps tiles [xs, xe) = [ceil((mu'_x + L - 15.5) / 16), floor((mu'_x + R - 0.5) / 16) + 1)
// inside the rectangle. Degenerate or extreme shapes (D <= 0, q >= 1e6, 2 s2 / D >= 1e30) keep
// the whole rectangle. Decisions in T (fp32 for parity), one op at a time.
// span gets 2 ints per rectangle row (xs, xe), xe == xs for an empty row. Returns the count.
// ---------------------------------------------------------------------------------------------
template <class T>
uint32_t tight_span(T mx, T my, T A, T B, T C, T o, const int32_t* rect, std::vector<int32_t>& span) {
  const int x0 = rect[0], y0 = rect[1], x1 = rect[2], y1 = rect[3];
  span.assign((size_t)2 * (size_t)std::max(y1 - y0, 0), 0);
  uint32_t cnt = 0;
  T kk = (T)2 * Act<T>::log((T)255 * o);
  if (!(kk > (T)0)) kk = (T)0;
  T k = std::sqrt(kk);
  if (k > (T)3.33) k = (T)3.33;
  const T s = (T)0.5 * k * k;
  const T D = A * C - B * B;
  const T q = (A * C) / D;
  bool full = !(A > (T)0) || !(C > (T)0) || !(D > (T)0) || !(q < (T)1e6);
  T s2 = (T)0, E = (T)0;
  if (!full) {
    s2 = s + ((T)0.002 + s * ((T)0.002 + q * ((T)1 / (T)65536)));
    E = (T)2 * s2 / D;
    full = !(E < (T)1e30);
  }
  for (int ty = y0; ty < y1; ++ty) {
    T xs = (T)x0, xe = (T)x1;
    if (!full) {
      const T ry = std::sqrt(E * A), t = std::sqrt(E / C);
      const T ylo = (T)(16 * ty) + (T)0.5 - my, yhi = (T)(16 * ty) + (T)15.5 - my;
      const T lo = std::max(ylo, -ry), hi = std::min(yhi, ry);
      if (lo > hi) {
        xs = xe = (T)x0;
      } else {
        const T vr = std::min(std::max(-(B * t), lo), hi);
        const T vl = std::min(std::max(B * t, lo), hi);
        const T R = (-(B * vr) + std::sqrt(std::max((T)2 * s2 * A - D * vr * vr, (T)0))) / A;
        const T L = (-(B * vl) - std::sqrt(std::max((T)2 * s2 * A - D * vl * vl, (T)0))) / A;
        xs = std::ceil((mx + L - (T)15.5) / (T)16);
        xe = std::floor((mx + R - (T)0.5) / (T)16) + (T)1;
        xs = std::min(std::max(xs, (T)x0), (T)x1);
        xe = std::min(std::max(xe, (T)x0), (T)x1);
        if (xe < xs) xe = xs;
      }
    }
    span[2 * (ty - y0)] = (int32_t)xs;
    span[2 * (ty - y0) + 1] = (int32_t)xe;
    cnt += (uint32_t)((int32_t)xe - (int32_t)xs);
  }
  return cnt;
}

template <class T>
void project_one(const T* mean, const T* log_scale, const T* quat, T logit, const T* sh,
                 int sh_degree, const Cam<T>& cam, Proj<T>& P) {
  std::memset(&P, 0, sizeof(P));
  P.defined = false;
  P.culled = true;
  const int K = (sh_degree + 1) * (sh_degree + 1);
  bool ok = finite(mean[0]) && finite(mean[1]) && finite(mean[2]) && finite(log_scale[0]) &&
            finite(log_scale[1]) && finite(log_scale[2]) && finite(quat[0]) && finite(quat[1]) &&
            finite(quat[2]) && finite(quat[3]) && finite(logit);
  for (int i = 0; i < K * 3 && ok; ++i) ok = finite(sh[i]);
  if (!ok) return;

  // Section 1: activations. q / max(|q|, 1e-12); s = exp(l); o = sigmoid(logit).
  T w = quat[0], x = quat[1], y = quat[2], z = quat[3];
  P.qn_raw = std::sqrt(((w * w + x * x) + y * y) + z * z);
  P.qn = std::max(P.qn_raw, (T)1e-12);
  w = w / P.qn; x = x / P.qn; y = y / P.qn; z = z / P.qn;
  P.q[0] = w; P.q[1] = x; P.q[2] = y; P.q[3] = z;
  for (int j = 0; j < 3; ++j) P.s[j] = Act<T>::exp(log_scale[j]);
  P.o = (T)1 / ((T)1 + Act<T>::exp(-logit));

  // Section 2: R(q) entry by entry, M = R diag(s) (column j times s_j), Sigma = M M^T.
  T* R = P.R;
  R[0] = (T)1 - (T)2 * (y * y + z * z);
  R[1] = (T)2 * (x * y - w * z);
  R[2] = (T)2 * (x * z + w * y);
  R[3] = (T)2 * (x * y + w * z);
  R[4] = (T)1 - (T)2 * (x * x + z * z);
  R[5] = (T)2 * (y * z - w * x);
  R[6] = (T)2 * (x * z - w * y);
  R[7] = (T)2 * (y * z + w * x);
  R[8] = (T)1 - (T)2 * (x * x + y * y);
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) P.M[i * 3 + j] = R[i * 3 + j] * P.s[j];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      P.Sig[i * 3 + j] = (P.M[i * 3 + 0] * P.M[j * 3 + 0] + P.M[i * 3 + 1] * P.M[j * 3 + 1]) +
                         P.M[i * 3 + 2] * P.M[j * 3 + 2];

  // Section 3: t = W mu + w0 and Sigma_c = W Sigma W^T with W the viewmat's rotation block.
  const T* V = cam.V;
  for (int r = 0; r < 3; ++r)
    P.t[r] = ((V[r * 4 + 0] * mean[0] + V[r * 4 + 1] * mean[1]) + V[r * 4 + 2] * mean[2]) + V[r * 4 + 3];
  T WS[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      WS[i * 3 + j] = (V[i * 4 + 0] * P.Sig[0 * 3 + j] + V[i * 4 + 1] * P.Sig[1 * 3 + j]) +
                      V[i * 4 + 2] * P.Sig[2 * 3 + j];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      P.Sc[i * 3 + j] = (WS[i * 3 + 0] * V[j * 4 + 0] + WS[i * 3 + 1] * V[j * 4 + 1]) +
                        WS[i * 3 + 2] * V[j * 4 + 2];
  const T tx = P.t[0], ty = P.t[1], tz = P.t[2];
  if (!(tz > cam.near_plane)) return;  // near cull (the "double where" example uses z > 0.01)

  // EWA Jacobian at the mean, its x/z and y/z clamped to the view widened by 0.3 tan(half-FoV)
  // on each side; the 2D mean itself is not clamped.
  const T fx = cam.fx, fy = cam.fy, cx = cam.cx, cy = cam.cy;
  const T tan_fovx = (T)0.5 * (T)cam.W / fx, tan_fovy = (T)0.5 * (T)cam.H / fy;
  const T lim_x_lo = -(cx / fx + (T)0.3 * tan_fovx), lim_x_hi = ((T)cam.W - cx) / fx + (T)0.3 * tan_fovx;
  const T lim_y_lo = -(cy / fy + (T)0.3 * tan_fovy), lim_y_hi = ((T)cam.H - cy) / fy + (T)0.3 * tan_fovy;
  P.xz = tx / tz;
  P.yz = ty / tz;
  P.clamp_x = (P.xz < lim_x_lo) || (P.xz > lim_x_hi);
  P.clamp_y = (P.yz < lim_y_lo) || (P.yz > lim_y_hi);
  P.jx = tz * std::min(std::max(P.xz, lim_x_lo), lim_x_hi);
  P.jy = tz * std::min(std::max(P.yz, lim_y_lo), lim_y_hi);
  T* J = P.J;
  J[0] = fx / tz; J[1] = (T)0; J[2] = -fx * P.jx / (tz * tz);
  J[3] = (T)0; J[4] = fy / tz; J[5] = -fy * P.jy / (tz * tz);

  // Sigma' = J Sigma_c J^T, then the eps2d low-pass: + 0.3 I (section 4).
  T JS[6];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 3; ++j)
      JS[i * 3 + j] = (J[i * 3 + 0] * P.Sc[0 * 3 + j] + J[i * 3 + 1] * P.Sc[1 * 3 + j]) +
                      J[i * 3 + 2] * P.Sc[2 * 3 + j];
  T C2[4];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      C2[i * 2 + j] = (JS[i * 3 + 0] * J[j * 3 + 0] + JS[i * 3 + 1] * J[j * 3 + 1]) + JS[i * 3 + 2] * J[j * 3 + 2];
  P.a = C2[0] + (T)0.3;
  P.b = C2[1];
  P.c = C2[3] + (T)0.3;
  P.det_raw = P.a * P.c - P.b * P.b;
  P.det = std::max(P.det_raw, (T)1e-10);
  P.a0 = C2[0];
  P.c0 = C2[3];
  P.det0 = C2[0] * C2[3] - C2[1] * C2[1];
  // Antialiased: o times sqrt(det Sigma2d / det Sigma'), which keeps the splat's integral
  // o 2 pi sqrt(det) equal to that of the undilated Gaussian (section 4's last variant).
  P.comp = cam.antialiased ? std::sqrt(std::max(P.det0, (T)0) / P.det) : (T)1;
  P.o_eff = cam.antialiased ? P.o * P.comp : P.o;
  P.conic[0] = P.c / P.det;
  P.conic[1] = -P.b / P.det;
  P.conic[2] = P.a / P.det;
  P.m2d[0] = fx * tx / tz + cx;
  P.m2d[1] = fy * ty / tz + cy;
  if (!(finite(P.a) && finite(P.b) && finite(P.c) && finite(P.conic[0]) && finite(P.conic[1]) &&
        finite(P.conic[2]) && finite(P.m2d[0]) && finite(P.m2d[1])))
    return;
  P.depth = tz;

  // Colour: sum_lm k_lm B_lm(d), d the unit vector from the camera centre to the mean.
  if (sh_degree == 0) {
    for (int ch = 0; ch < 3; ++ch) P.color[ch] = sh[ch];
  } else {
    T C[3];
    for (int j = 0; j < 3; ++j) C[j] = -((V[0 * 4 + j] * V[3] + V[1 * 4 + j] * V[7]) + V[2 * 4 + j] * V[11]);
    T d[3] = {mean[0] - C[0], mean[1] - C[1], mean[2] - C[2]};
    P.dir_norm = std::sqrt((d[0] * d[0] + d[1] * d[1]) + d[2] * d[2]);
    T dn = std::max(P.dir_norm, (T)1e-12);
    for (int j = 0; j < 3; ++j) P.dir[j] = d[j] / dn;
    T B[16];
    sh_basis<T>(sh_degree, P.dir[0], P.dir[1], P.dir[2], B);
    for (int ch = 0; ch < 3; ++ch) {
      T acc = (T)0;
      for (int l = 0; l < K; ++l) acc = acc + sh[l * 3 + ch] * B[l];
      P.color[ch] = acc;
    }
  }
  P.defined = true;

  // The original 3DGS radius, ceil(3 sqrt(lambda_max)) with the root's argument floored at 0.1,
  // reported alongside (it is not used for binning).
  T mid = (T)0.5 * (P.a + P.c);
  T lam = mid + std::sqrt(std::max(mid * mid - P.det, (T)0.1));
  const T sat3 = (T)16777216;
  P.radius_3dgs = (int)std::min(std::ceil((T)3 * std::sqrt(lam)), sat3);

  // Radius: per-axis extent of the k-sigma ellipse, k = min(3.33, sqrt(2 ln(255 o))): the
  // distance at which o exp(-m^2/2) falls below 1/255 (o the opacity the blend uses).
  // Gaussians with o < 1/255 never reach it. With radius_mode 1 both radii are the 3DGS one.
  if (P.o_eff < (T)1 / (T)255) return;
  T kk = (T)2 * Act<T>::log((T)255 * P.o_eff);
  if (!(kk > (T)0)) kk = (T)0;
  P.k = std::sqrt(kk);
  if (P.k > (T)3.33) P.k = (T)3.33;
  const T sat = (T)16777216;  // 2^24: radii are saturated here (far beyond any tile grid)
  if (cam.radius_mode == 1) {
    P.rx = P.ry = (T)P.radius_3dgs;
  } else {
    P.rx = std::min(std::ceil(P.k * std::sqrt(P.a)), sat);
    P.ry = std::min(std::ceil(P.k * std::sqrt(P.c)), sat);
  }

  // Tile rectangle [floor((mu - r)/16), ceil((mu + r)/16)) clamped to the grid.
  T x0 = std::floor((P.m2d[0] - P.rx) / (T)16), x1 = std::ceil((P.m2d[0] + P.rx) / (T)16);
  T y0 = std::floor((P.m2d[1] - P.ry) / (T)16), y1 = std::ceil((P.m2d[1] + P.ry) / (T)16);
  x0 = std::min(std::max(x0, (T)0), (T)cam.tiles_x);
  x1 = std::min(std::max(x1, (T)0), (T)cam.tiles_x);
  y0 = std::min(std::max(y0, (T)0), (T)cam.tiles_y);
  y1 = std::min(std::max(y1, (T)0), (T)cam.tiles_y);
  P.rect[0] = (int)x0; P.rect[1] = (int)y0; P.rect[2] = (int)x1; P.rect[3] = (int)y1;
  if (!(P.rect[2] > P.rect[0] && P.rect[3] > P.rect[1])) return;  // nothing on screen
  P.tiles = (uint32_t)((P.rect[2] - P.rect[0]) * (P.rect[3] - P.rect[1]));
  if (cam.tight_tiles) {
    std::vector<int32_t> span;
    P.tiles = tight_span<T>(P.m2d[0], P.m2d[1], P.conic[0], P.conic[1], P.conic[2], P.o_eff, P.rect, span);
    if (P.tiles == 0) return;  // the ellipse reaches no pixel centre
  }

  P.culled = false;
}

// ---------------------------------------------------------------------------------------------
// Per-pixel trace of the blend (section 5's loop), decisions in T.
// ---------------------------------------------------------------------------------------------
template <class T> struct Splat2D {
  T mx, my, A, B, C, o, col[3];
  T z;           // camera depth: the value the depth channel blends
  T skip_above;  // ln(255 o) + 1e-3: sigma above this implies alpha < 1/255 (exact shortcut)
  std::vector<int32_t> span;  // tight tile rows (xs, xe) per rectangle row; empty: whole rectangle
};

struct Contributor {
  int g;        // Gaussian id
  bool capped;  // alpha hit the 0.99 cap
};

struct Trace {
  std::vector<Contributor> contrib;
  bool fragile = false;
  double errT = 0.0;  // bound on the relative rounding of the final transmittance (band units)
  int64_t n_eval = 0;
  int64_t escapes = 0;
};

// Walks `order` (un-culled Gaussians, stable ascending depth) at pixel centre (px, py).
// fragile is set when a decision lies within the rounding band of its threshold. band_eps is the
// unit roundoff of the implementation being compared (2^-24 for fp32); the band of each compared
// quantity is a bound on its accumulated relative rounding, with a safety factor of 8:
//   sigma: 8 eps times the sum of the magnitudes of its terms,
//   alpha: that (relative, through exp) plus 8 eps,
//   T * (1 - alpha): the running bound on T plus alpha / (1 - alpha) times alpha's bound.
template <class T>
void trace_pixel(T px, T py, const std::vector<int>& order, const std::vector<Splat2D<T>>& S,
                 const int32_t* rects, int tile_x, int tile_y, double band_eps, Trace& tr) {
  tr.contrib.clear();
  tr.fragile = false;
  tr.n_eval = 0;
  tr.escapes = 0;
  tr.errT = 0.0;
  T Tr = (T)1;
  double errT = 0.0;  // bound on the relative rounding carried by Tr, in units of band_eps
  const T thr_a = (T)1 / (T)255;
  for (int g : order) {
    const Splat2D<T>& s = S[g];
    T dx = s.mx - px, dy = s.my - py;
    T sigma = (T)0.5 * (s.A * dx * dx + s.C * dy * dy) + s.B * dx * dy;
    // Exact shortcut: sigma > ln(255 o) + 1e-3 implies o e^-sigma < (1/255) e^-0.001, a skip
    // whatever the rounding; it changes no decision and only saves the exponential.
    if (sigma > s.skip_above) continue;
    ++tr.n_eval;
    T G = (T)std::exp(-(double)sigma);
    T raw = s.o * G;
    T alpha = std::min((T)0.99, raw);
    // rounding bound on sigma (relative to the magnitudes summed) and on alpha
    double sig_mag = 0.5 * (std::fabs((double)s.A) * dx * dx + std::fabs((double)s.C) * dy * dy) +
                     std::fabs((double)s.B * dx * dy);
    double e_sig = 8.0 * band_eps * sig_mag;   // absolute, on sigma
    double e_alpha = e_sig + 8.0 * band_eps;   // relative, on alpha
    // The tiled renderer's lists: a pixel sees only the Gaussians whose tile rectangle holds its
    // tile. One outside that would pass the skip test is counted as an escape (a difference from
    // the dense render; none with the opacity-aware radius) and then ignored.
    bool inside = tile_x >= rects[g * 4 + 0] && tile_x < rects[g * 4 + 2] &&
                  tile_y >= rects[g * 4 + 1] && tile_y < rects[g * 4 + 3];
    if (inside && !s.span.empty()) {
      const int r = tile_y - rects[g * 4 + 1];
      inside = tile_x >= s.span[2 * r] && tile_x < s.span[2 * r + 1];
    }
    if (!inside) {
      if (!(sigma < (T)0 || alpha < thr_a)) ++tr.escapes;
      continue;
    }
    if (std::fabs((double)sigma) <= e_sig) tr.fragile = true;
    if (std::fabs((double)alpha - (double)thr_a) <= e_alpha * (double)thr_a) tr.fragile = true;
    if (std::fabs((double)raw - 0.99) <= e_alpha * 0.99) tr.fragile = true;
    if (sigma < (T)0 || alpha < thr_a) continue;
    // contributes unless it would drive T to or below 1e-4
    T next_T = Tr * ((T)1 - alpha);
    double errN = errT + e_alpha * (double)alpha / (1.0 - (double)alpha) + 2.0 * band_eps;
    if (std::fabs((double)next_T - 1e-4) <= errN * 1e-4) tr.fragile = true;
    if (next_T <= (T)1e-4) break;
    tr.contrib.push_back({g, raw >= (T)0.99});
    Tr = next_T;
    errT = errN;
    tr.errT = errT;
  }
}

template <class T>
void build_splats(int n, const T* means2d, const T* conics, const T* opac, const T* colors,
                  const T* depths, const uint32_t* tiles, const int32_t* rects, int tight,
                  std::vector<Splat2D<T>>& S, std::vector<int>& order) {
  S.resize(n);
  order.clear();
  for (int g = 0; g < n; ++g) {
    S[g] = {means2d[2 * g], means2d[2 * g + 1], conics[3 * g], conics[3 * g + 1], conics[3 * g + 2],
            opac[g], {colors[3 * g], colors[3 * g + 1], colors[3 * g + 2]}, depths[g], (T)0, {}};
    S[g].skip_above = opac[g] > (T)0 ? (T)(std::log(255.0 * (double)opac[g]) + 1e-3) : (T)0;
    if (tiles[g] > 0) order.push_back(g);
    if (tight && tiles[g] > 0)
      tight_span<T>(S[g].mx, S[g].my, S[g].A, S[g].B, S[g].C, S[g].o, rects + 4 * g, S[g].span);
  }
  // one global, stable ascending-depth order (ties keep ascending Gaussian id)
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return depths[a] < depths[b]; });
}

int nthreads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
int thread_id() {
#ifdef _OPENMP
  return omp_get_thread_num();
#else
  return 0;
#endif
}

// Pixel list: npix pairs (row, col); NULL means every pixel in row-major order.
inline void pixel_of(const int32_t* pix, int W, int64_t p, int& row, int& col) {
  if (pix) {
    row = pix[2 * p];
    col = pix[2 * p + 1];
  } else {
    row = (int)(p / W);
    col = (int)(p % W);
  }
}

// Values of one traced pixel, in double: alpha_i, T_i (transmittance in front of i) and G_i.
template <class T>
void pixel_values(const Trace& tr, const std::vector<Splat2D<T>>& S, double px, double py,
                  std::vector<double>& al, std::vector<double>& Ti, std::vector<double>& Gi,
                  double& T_final) {
  size_t n = tr.contrib.size();
  al.resize(n); Ti.resize(n); Gi.resize(n);
  double Tr = 1.0;
  for (size_t i = 0; i < n; ++i) {
    const Splat2D<T>& s = S[tr.contrib[i].g];
    double dx = (double)s.mx - px, dy = (double)s.my - py;
    double sigma = 0.5 * ((double)s.A * dx * dx + (double)s.C * dy * dy) + (double)s.B * dx * dy;
    Gi[i] = std::exp(-sigma);
    al[i] = tr.contrib[i].capped ? 0.99 : (double)s.o * Gi[i];
    Ti[i] = Tr;
    Tr = Tr * (1.0 - al[i]);
  }
  T_final = Tr;
}

template <class T>
int render_impl(int n, const T* means2d, const T* conics, const T* opac, const T* colors,
                const T* depths, const uint32_t* tiles, const int32_t* rects, int tight, int W, int H,
                const T* bg, int64_t npix, const int32_t* pix, double band_eps, double* image,
                double* final_T, int32_t* last_id, int32_t* n_contrib, uint8_t* fragile,
                int64_t* escapes, int64_t* n_eval, double* depth_img) {
  std::vector<Splat2D<T>> S;
  std::vector<int> order;
  build_splats<T>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, S, order);
  if (!pix) npix = (int64_t)W * H;
  int64_t esc = 0, nev = 0;
#pragma omp parallel reduction(+ : esc, nev)
  {
    Trace tr;
    std::vector<double> al, Ti, Gi;
#pragma omp for schedule(dynamic, 16)
    for (int64_t p = 0; p < npix; ++p) {
      int row, col;
      pixel_of(pix, W, p, row, col);
      T px = (T)col + (T)0.5, py = (T)row + (T)0.5;
      trace_pixel<T>(px, py, order, S, rects, col / 16, row / 16, band_eps, tr);
      double Tf;
      pixel_values<T>(tr, S, (double)px, (double)py, al, Ti, Gi, Tf);
      double acc[3] = {0, 0, 0};
      for (size_t i = 0; i < tr.contrib.size(); ++i)
        for (int ch = 0; ch < 3; ++ch) acc[ch] += (double)S[tr.contrib[i].g].col[ch] * al[i] * Ti[i];
      for (int ch = 0; ch < 3; ++ch) image[3 * p + ch] = acc[ch] + Tf * (double)bg[ch];
      if (depth_img) {
        // the depth channel: camera z blended with the same weights, background depth 0
        double d = 0.0;
        for (size_t i = 0; i < tr.contrib.size(); ++i) d += (double)S[tr.contrib[i].g].z * al[i] * Ti[i];
        depth_img[p] = d;
      }
      final_T[p] = Tf;
      last_id[p] = tr.contrib.empty() ? -1 : tr.contrib.back().g;
      n_contrib[p] = (int32_t)tr.contrib.size();
      fragile[p] = tr.fragile ? 1 : 0;
      esc += tr.escapes;
      nev += tr.n_eval;
    }
  }
  *escapes = esc;
  *n_eval = nev;
  return 0;
}

// Backward of the blend (per pixel, back to front in the plain suffix-sum form):
//   C = sum_i c_i a_i T_i + T_final bg,
//   dC/dc_i = a_i T_i,  dC/da_i = c_i T_i - S_i / (1 - a_i),  S_i = sum_{j>i} c_j a_j T_j + T_final bg,
//   a = o exp(-sigma) when below the cap (else constant 0.99): da/do = exp(-sigma), da/dsigma = -a,
//   sigma = 0.5 (A dx^2 + C dy^2) + B dx dy with dx = mu'_x - px.
// With a depth channel (dL_ddepth, may be NULL) its value z_i joins the colours: D = sum_i z_i a_i T_i
// (background depth 0), so dD/dz_i = a_i T_i and dD/da_i = z_i T_i - S^D_i / (1 - a_i).
// Output per Gaussian (10): d mu'_x, d mu'_y, dA, dB, dC, d opacity, d colour (3), d depth,
// accumulated in double. Two rounding scales of each sum, for tolerance floors:
//   aref_plain: the sum over pixels of the absolute per-pixel contribution |dC_p/d.| (may be NULL);
//   aref_terms: aref without the widening by the transmittance's rounding bound (may be NULL);
//   aref: per pixel, the absolute values of the terms each contribution is computed from (|c| T +
//     |S| / (1 - a) for dC/da, which cancels when a splat's colour matches what lies behind it),
//     times max(1, e_T / 1e-5) with e_T the pixel's bound on the relative rounding of its
//     transmittance, summed over pixels (may be NULL).
template <class T>
int render_bwd_impl(int n, const T* means2d, const T* conics, const T* opac, const T* colors,
                    const T* depths, const uint32_t* tiles, const int32_t* rects, int tight, int W, int H,
                    const T* bg, int64_t npix, const int32_t* pix, double band_eps,
                    const double* dL_dimg, const double* dL_ddepth, double* g2d, double* aref,
                    double* aref_plain, double* aref_terms) {
  std::vector<Splat2D<T>> S;
  std::vector<int> order;
  build_splats<T>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, S, order);
  if (!pix) npix = (int64_t)W * H;
  const int nt = nthreads();
  std::vector<std::vector<double>> accg(nt), acca(nt), accp(nt), acct(nt);
#pragma omp parallel
  {
    const int tid = thread_id();
    accg[tid].assign((size_t)n * 10, 0.0);
    acca[tid].assign((size_t)n * 10, 0.0);
    accp[tid].assign((size_t)n * 10, 0.0);
    acct[tid].assign((size_t)n * 10, 0.0);
    double* G = accg[tid].data();
    double* Aa = acca[tid].data();
    double* Ap = accp[tid].data();
    double* At = acct[tid].data();
    Trace tr;
    std::vector<double> al, Ti, Gi;
#pragma omp for schedule(dynamic, 16)
    for (int64_t p = 0; p < npix; ++p) {
      const double* gp = dL_dimg + 3 * p;
      const double gd = dL_ddepth ? dL_ddepth[p] : 0.0;
      if (gp[0] == 0.0 && gp[1] == 0.0 && gp[2] == 0.0 && gd == 0.0) continue;
      int row, col;
      pixel_of(pix, W, p, row, col);
      T px = (T)col + (T)0.5, py = (T)row + (T)0.5;
      trace_pixel<T>(px, py, order, S, rects, col / 16, row / 16, band_eps, tr);
      double Tf;
      pixel_values<T>(tr, S, (double)px, (double)py, al, Ti, Gi, Tf);
      // T_i is recovered from rounded (1 - alpha) factors: where the bound on its relative rounding
      // exceeds 1e-5, the floor of this pixel's terms grows with it
      const double tscale = std::max(1.0, tr.errT / 1e-5);
      double Sacc[3] = {Tf * (double)bg[0], Tf * (double)bg[1], Tf * (double)bg[2]};
      double Sabs[3] = {Tf * std::fabs((double)bg[0]), Tf * std::fabs((double)bg[1]), Tf * std::fabs((double)bg[2])};
      double SD = 0.0, SDabs = 0.0;  // the depth channel's S (background depth 0)
      for (int i = (int)tr.contrib.size() - 1; i >= 0; --i) {
        const int g = tr.contrib[i].g;
        const Splat2D<T>& s = S[g];
        double c[3] = {(double)s.col[0], (double)s.col[1], (double)s.col[2]};
        double gal = 0.0, gal_mag = 0.0;
        for (int ch = 0; ch < 3; ++ch) {
          gal += gp[ch] * (c[ch] * Ti[i] - Sacc[ch] / (1.0 - al[i]));
          gal_mag += std::fabs(gp[ch]) * (std::fabs(c[ch]) * Ti[i] + Sabs[ch] / (1.0 - al[i]));
        }
        const double z = (double)s.z;
        gal += gd * (z * Ti[i] - SD / (1.0 - al[i]));
        gal_mag += std::fabs(gd) * (std::fabs(z) * Ti[i] + SDabs / (1.0 - al[i]));
        double contrib[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0}, mag[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        for (int ch = 0; ch < 3; ++ch) {
          contrib[6 + ch] = al[i] * Ti[i] * gp[ch];
          mag[6 + ch] = std::fabs(contrib[6 + ch]);
        }
        contrib[9] = al[i] * Ti[i] * gd;
        mag[9] = std::fabs(contrib[9]);
        if (!tr.contrib[i].capped) {
          double dx = (double)s.mx - (double)px, dy = (double)s.my - (double)py;
          contrib[5] = Gi[i] * gal;
          double gsig = -al[i] * gal;
          double dsig[5] = {(double)s.A * dx + (double)s.B * dy, (double)s.B * dx + (double)s.C * dy,
                            0.5 * dx * dx, dx * dy, 0.5 * dy * dy};
          for (int k = 0; k < 5; ++k) contrib[k] = gsig * dsig[k];
          // magnitudes: dC/dalpha summed from its terms' absolute values; d sigma/d mean2d too
          mag[5] = Gi[i] * gal_mag;
          double dsig_mag[5] = {std::fabs((double)s.A * dx) + std::fabs((double)s.B * dy),
                                std::fabs((double)s.B * dx) + std::fabs((double)s.C * dy), std::fabs(dsig[2]),
                                std::fabs(dsig[3]), std::fabs(dsig[4])};
          for (int k = 0; k < 5; ++k) mag[k] = al[i] * gal_mag * dsig_mag[k];
        }
        for (int k = 0; k < 10; ++k) {
          G[(size_t)g * 10 + k] += contrib[k];
          Aa[(size_t)g * 10 + k] += mag[k] * tscale;
          Ap[(size_t)g * 10 + k] += std::fabs(contrib[k]);
          At[(size_t)g * 10 + k] += mag[k];
        }
        for (int ch = 0; ch < 3; ++ch) {
          Sacc[ch] += c[ch] * al[i] * Ti[i];
          Sabs[ch] += std::fabs(c[ch]) * al[i] * Ti[i];
        }
        SD += z * al[i] * Ti[i];
        SDabs += std::fabs(z) * al[i] * Ti[i];
      }
    }
  }
  for (size_t i = 0; i < (size_t)n * 10; ++i) {
    double sg = 0, sa = 0, sp = 0, st = 0;
    for (int t = 0; t < nt; ++t) {
      sg += accg[t][i];
      sa += acca[t][i];
      sp += accp[t][i];
      st += acct[t][i];
    }
    g2d[i] = sg;
    if (aref) aref[i] = sa;
    if (aref_plain) aref_plain[i] = sp;
    if (aref_terms) aref_terms[i] = st;
  }
  return 0;
}

// Backward of the projection for one Gaussian, in double, given the decisions (cull, clamps,
// det clamp, near) of the T-precision forward. g9 = (d mu'_x, d mu'_y, dA, dB, dC, d o, d rgb,
// d depth): 10 values, the depth being camera z = t_z.
void project_bwd_one(const double* mean, const double* log_scale, const double* quat, double logit,
                     const double* sh, int sh_degree, const Cam<double>& cam, bool clamp_x,
                     bool clamp_y, bool det_clamped, const double* g9, double* d_mean,
                     double* d_log_scale, double* d_quat, double* d_logit, double* d_sh) {
  Proj<double> P;
  project_one<double>(mean, log_scale, quat, logit, sh, sh_degree, cam, P);
  const int K = (sh_degree + 1) * (sh_degree + 1);
  const double a = P.a, b = P.b, c = P.c;
  const double det = det_clamped ? 1e-10 : a * c - b * b;
  // conic (A, B, C) = (c, -b, a) / det
  const double gA = g9[2], gB = g9[3], gC = g9[4];
  double ga, gb, gc;
  if (det_clamped) {
    ga = gC / det; gb = -gB / det; gc = gA / det;
  } else {
    const double d2 = det * det;
    // d det/da = c, d det/db = -2b, d det/dc = a
    ga = gA * (-c * c / d2) + gB * (b * c / d2) + gC * (1.0 / det - a * c / d2);
    gb = gA * (2.0 * b * c / d2) + gB * (-1.0 / det - 2.0 * b * b / d2) + gC * (2.0 * a * b / d2);
    gc = gA * (1.0 / det - a * c / d2) + gB * (a * b / d2) + gC * (-a * a / d2);
  }
  if (cam.antialiased && P.comp > 0.0) {
    // o_eff = o comp, comp = sqrt(det0 / det): d comp = comp / 2 (d det0 / det0 - d det / det),
    // det0 = a0 c0 - b^2 and det = a c - b^2 with a = a0 + 0.3, c = c0 + 0.3 (da = da0)
    const double h = 0.5 * g9[5] * P.o * P.comp, det0 = P.det0;
    ga += h * (P.c0 / det0 - c / det);
    gc += h * (P.a0 / det0 - a / det);
    gb += h * (-2.0 * b / det0 + 2.0 * b / det);
  }
  // Sigma' = J Sc J^T + 0.3 I with entries (a, b; b, c): symmetric gradient G2.
  double G2[4] = {ga, 0.5 * gb, 0.5 * gb, gc};
  const double* J = P.J;
  const double* Sc = P.Sc;
  // dL/dSc = J^T G2 J (3x3)
  double gSc[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int p = 0; p < 2; ++p)
        for (int q = 0; q < 2; ++q) acc += J[p * 3 + i] * G2[p * 2 + q] * J[q * 3 + j];
      gSc[i * 3 + j] = acc;
    }
  // dL/dJ = 2 G2 J Sc (2x3)
  double gJ[6];
  for (int p = 0; p < 2; ++p)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int q = 0; q < 2; ++q)
        for (int k = 0; k < 3; ++k) acc += 2.0 * G2[p * 2 + q] * J[q * 3 + k] * Sc[k * 3 + j];
      gJ[p * 3 + j] = acc;
    }
  const double tx = P.t[0], ty = P.t[1], tz = P.t[2];
  const double fx = cam.fx, fy = cam.fy;
  double gt[3] = {0, 0, 0};
  // J00 = fx/tz, J11 = fy/tz
  gt[2] += gJ[0] * (-fx / (tz * tz)) + gJ[4] * (-fy / (tz * tz));
  // J02 = -fx jx / tz^2 with jx = tx (unclamped) or tz * L (clamped)
  {
    const double dj_dtx = clamp_x ? 0.0 : 1.0, dj_dtz = clamp_x ? P.jx / tz : 0.0;
    gt[0] += gJ[2] * (-fx / (tz * tz)) * dj_dtx;
    gt[2] += gJ[2] * (2.0 * fx * P.jx / (tz * tz * tz) - fx * dj_dtz / (tz * tz));
    const double dk_dty = clamp_y ? 0.0 : 1.0, dk_dtz = clamp_y ? P.jy / tz : 0.0;
    gt[1] += gJ[5] * (-fy / (tz * tz)) * dk_dty;
    gt[2] += gJ[5] * (2.0 * fy * P.jy / (tz * tz * tz) - fy * dk_dtz / (tz * tz));
  }
  // mu' = (fx tx/tz + cx, fy ty/tz + cy)
  gt[0] += g9[0] * fx / tz;
  gt[2] += -g9[0] * fx * tx / (tz * tz);
  gt[1] += g9[1] * fy / tz;
  gt[2] += -g9[1] * fy * ty / (tz * tz);
  // the depth channel's value is t_z
  gt[2] += g9[9];
  // t = W mu + w0  ->  dL/dmu = W^T dL/dt;  Sc = W Sig W^T  ->  dL/dSig = W^T dL/dSc W
  const double* V = cam.V;
  for (int j = 0; j < 3; ++j) d_mean[j] = V[0 * 4 + j] * gt[0] + V[1 * 4 + j] * gt[1] + V[2 * 4 + j] * gt[2];
  double gSig[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int p = 0; p < 3; ++p)
        for (int q = 0; q < 3; ++q) acc += V[p * 4 + i] * gSc[p * 3 + q] * V[q * 4 + j];
      gSig[i * 3 + j] = acc;
    }
  // Sig = M M^T -> dL/dM = (gSig + gSig^T) M
  double gM[9];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += (gSig[i * 3 + k] + gSig[k * 3 + i]) * P.M[k * 3 + j];
      gM[i * 3 + j] = acc;
    }
  // M = R diag(s)
  double gR[9], gs[3] = {0, 0, 0};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      gR[i * 3 + j] = gM[i * 3 + j] * P.s[j];
      gs[j] += gM[i * 3 + j] * P.R[i * 3 + j];
    }
  for (int j = 0; j < 3; ++j) d_log_scale[j] = gs[j] * P.s[j];
  // R(q) with q = (w, x, y, z) normalised: derivatives of the nine entries
  const double w = P.q[0], x = P.q[1], y = P.q[2], z = P.q[3];
  double gq[4];
  gq[0] = 2.0 * (-z * gR[1] + y * gR[2] + z * gR[3] - x * gR[5] - y * gR[6] + x * gR[7]);
  gq[1] = 2.0 * (y * gR[1] + z * gR[2] + y * gR[3] - 2.0 * x * gR[4] - w * gR[5] + z * gR[6] + w * gR[7] -
                 2.0 * x * gR[8]);
  gq[2] = 2.0 * (-2.0 * y * gR[0] + x * gR[1] + w * gR[2] + x * gR[3] + z * gR[5] - w * gR[6] + z * gR[7] -
                 2.0 * y * gR[8]);
  gq[3] = 2.0 * (-2.0 * z * gR[0] - w * gR[1] + x * gR[2] + w * gR[3] - 2.0 * z * gR[4] + y * gR[5] +
                 x * gR[6] + y * gR[7]);
  // q_hat = q / max(|q|, 1e-12)
  if (P.qn_raw > 1e-12) {
    double dot = w * gq[0] + x * gq[1] + y * gq[2] + z * gq[3];
    for (int j = 0; j < 4; ++j) d_quat[j] = (gq[j] - P.q[j] * dot) / P.qn;
  } else {
    for (int j = 0; j < 4; ++j) d_quat[j] = gq[j] / P.qn;
  }
  // o = sigmoid(logit); the blend's opacity is o comp
  *d_logit = P.o * (1.0 - P.o) * P.comp * g9[5];
  // colour
  if (sh_degree == 0) {
    for (int ch = 0; ch < 3; ++ch) d_sh[ch] = g9[6 + ch];
  } else {
    double B[16];
    sh_basis<double>(sh_degree, P.dir[0], P.dir[1], P.dir[2], B);
    for (int l = 0; l < K; ++l)
      for (int ch = 0; ch < 3; ++ch) d_sh[l * 3 + ch] = B[l] * g9[6 + ch];
    double dB[16][3];
    sh_basis_grad(sh_degree, P.dir[0], P.dir[1], P.dir[2], dB);
    double gd[3] = {0, 0, 0};
    for (int l = 1; l < K; ++l)
      for (int ch = 0; ch < 3; ++ch) {
        double wgt = sh[l * 3 + ch] * g9[6 + ch];
        for (int j = 0; j < 3; ++j) gd[j] += wgt * dB[l][j];
      }
    double dot = P.dir[0] * gd[0] + P.dir[1] * gd[1] + P.dir[2] * gd[2];
    double dn = std::max(P.dir_norm, 1e-12);
    for (int j = 0; j < 3; ++j) d_mean[j] += (gd[j] - P.dir[j] * dot) / dn;
  }
}

template <class T>
int project_impl(int n, int sh_degree, const T* means, const T* log_scales, const T* quats,
                 const T* logits, const T* sh, const T* camp, int W, int H, T* means2d, T* conics,
                 T* depths, int32_t* radii, T* opac, T* colors, int32_t* rects, uint32_t* tiles,
                 T* cov2d, int32_t* radius_3dgs) {
  if (sh_degree < 0 || sh_degree > 3) return 1;
  Cam<T> cam = make_cam<T>(camp, W, H);
  const int K = (sh_degree + 1) * (sh_degree + 1);
#pragma omp parallel for schedule(static)
  for (int g = 0; g < n; ++g) {
    Proj<T> P;
    project_one<T>(means + 3 * g, log_scales + 3 * g, quats + 4 * g, logits[g], sh + (size_t)g * K * 3,
                   sh_degree, cam, P);
    // Undefined projections (behind the near plane, non-finite) write zeros; defined ones
    // write their projected values, and radii/rect/tiles stay 0 unless the Gaussian is drawn.
    means2d[2 * g] = P.m2d[0];
    means2d[2 * g + 1] = P.m2d[1];
    for (int j = 0; j < 3; ++j) conics[3 * g + j] = P.conic[j];
    depths[g] = P.depth;
    opac[g] = P.o_eff;
    for (int j = 0; j < 3; ++j) colors[3 * g + j] = P.color[j];
    if (cov2d) {
      cov2d[3 * g] = P.a;
      cov2d[3 * g + 1] = P.b;
      cov2d[3 * g + 2] = P.c;
    }
    if (radius_3dgs) radius_3dgs[g] = P.radius_3dgs;
    if (!P.defined) {
      means2d[2 * g] = means2d[2 * g + 1] = (T)0;
      for (int j = 0; j < 3; ++j) conics[3 * g + j] = colors[3 * g + j] = (T)0;
      depths[g] = opac[g] = (T)0;
      if (cov2d) cov2d[3 * g] = cov2d[3 * g + 1] = cov2d[3 * g + 2] = (T)0;
      if (radius_3dgs) radius_3dgs[g] = 0;
    }
    const bool drawn = !P.culled;
    radii[2 * g] = drawn ? (int32_t)P.rx : 0;
    radii[2 * g + 1] = drawn ? (int32_t)P.ry : 0;
    for (int j = 0; j < 4; ++j) rects[4 * g + j] = drawn ? P.rect[j] : 0;
    tiles[g] = drawn ? P.tiles : 0u;
  }
  return 0;
}

template <class T>
int project_bwd_impl(int n, int sh_degree, const T* means, const T* log_scales, const T* quats,
                     const T* logits, const T* sh, const T* camp, int W, int H, const double* g2d,
                     const double* aref2d, double* d_means, double* d_log_scales, double* d_quats,
                     double* d_logits, double* d_sh, double* aref_raw) {
  if (sh_degree < 0 || sh_degree > 3) return 1;
  Cam<T> cam = make_cam<T>(camp, W, H);
  double cp[kNumCam];
  for (int i = 0; i < kNumCam; ++i) cp[i] = (double)camp[i];
  Cam<double> camd = make_cam<double>(cp, W, H);
  const int K = (sh_degree + 1) * (sh_degree + 1);
  const int nraw = 3 + 3 + 4 + 1 + K * 3;
#pragma omp parallel for schedule(static)
  for (int g = 0; g < n; ++g) {
    Proj<T> P;
    project_one<T>(means + 3 * g, log_scales + 3 * g, quats + 4 * g, logits[g], sh + (size_t)g * K * 3,
                   sh_degree, cam, P);
    double* dm = d_means + 3 * g;
    double* dl = d_log_scales + 3 * g;
    double* dq = d_quats + 4 * g;
    double* dsh = d_sh + (size_t)g * K * 3;
    for (int j = 0; j < 3; ++j) dm[j] = dl[j] = 0.0;
    for (int j = 0; j < 4; ++j) dq[j] = 0.0;
    d_logits[g] = 0.0;
    for (int j = 0; j < K * 3; ++j) dsh[j] = 0.0;
    if (aref_raw)
      for (int j = 0; j < nraw; ++j) aref_raw[(size_t)g * nraw + j] = 0.0;
    if (P.culled) continue;  // culled Gaussians get exactly zero gradient
    double mean[3], ls[3], q[4], lg = (double)logits[g];
    for (int j = 0; j < 3; ++j) {
      mean[j] = (double)means[3 * g + j];
      ls[j] = (double)log_scales[3 * g + j];
    }
    for (int j = 0; j < 4; ++j) q[j] = (double)quats[4 * g + j];
    std::vector<double> shd(K * 3);
    for (int j = 0; j < K * 3; ++j) shd[j] = (double)sh[(size_t)g * K * 3 + j];
    const bool det_clamped = !(P.det_raw >= (T)1e-10);
    project_bwd_one(mean, ls, q, lg, shd.data(), sh_degree, camd, P.clamp_x, P.clamp_y, det_clamped,
                    g2d + 10 * (size_t)g, dm, dl, dq, d_logits + g, dsh);
    if (aref_raw && aref2d) {
      // floor for the raw gradients: |Jacobian| applied to the 2D absolute sums
      double* ar = aref_raw + (size_t)g * nraw;
      std::vector<double> tmp(nraw);
      for (int k = 0; k < 10; ++k) {
        double e[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        e[k] = 1.0;
        double tl;
        project_bwd_one(mean, ls, q, lg, shd.data(), sh_degree, camd, P.clamp_x, P.clamp_y, det_clamped, e,
                        tmp.data(), tmp.data() + 3, tmp.data() + 6, &tl, tmp.data() + 11);
        tmp[10] = tl;
        for (int j = 0; j < nraw; ++j) ar[j] += std::fabs(tmp[j]) * aref2d[10 * (size_t)g + k];
      }
    }
  }
  return 0;
}

}  // namespace

extern "C" {

// -- D1 functions, elementwise ------------------------------------------------------------------
void orc_exp_f32(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = d1_expf(x[i]);
}
void orc_log_f32(const float* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = d1_logf(x[i]);
}

// -- single steps, exposed for pins ---------------------------------------------------------------
// quaternion (w,x,y,z) and log-scales -> normalised R [9] and Sigma [9]
void orc_covariance_f64(const double* quat, const double* log_scale, double* R, double* Sigma) {
  // identity view, unit focal lengths, near 0.01, black background, default options
  double cam[kNumCam] = {1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 1, 1, 0, 0, 0.01, 0, 0, 0, 0, 0, 0};
  double mean[3] = {0, 0, 1}, sh[3] = {0, 0, 0};
  Proj<double> P;
  Cam<double> c = make_cam<double>(cam, 1, 1);
  project_one<double>(mean, log_scale, quat, 0.0, sh, 0, c, P);
  for (int i = 0; i < 9; ++i) {
    R[i] = P.R[i];
    Sigma[i] = P.Sig[i];
  }
}
void orc_sh_basis_f64(int degree, const double* dirs, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    double B[16] = {0};
    sh_basis<double>(degree, dirs[3 * i], dirs[3 * i + 1], dirs[3 * i + 2], B);
    for (int k = 0; k < 16; ++k) out[16 * i + k] = B[k];
  }
}

// -- projection -------------------------------------------------------------------------------------
int orc_project_f32(int n, int sh_degree, const float* means, const float* log_scales, const float* quats,
                    const float* logits, const float* sh, const float* cam, int W, int H, float* means2d,
                    float* conics, float* depths, int32_t* radii, float* opac, float* colors, int32_t* rects,
                    uint32_t* tiles, float* cov2d, int32_t* radius_3dgs) {
  return project_impl<float>(n, sh_degree, means, log_scales, quats, logits, sh, cam, W, H, means2d, conics,
                             depths, radii, opac, colors, rects, tiles, cov2d, radius_3dgs);
}
int orc_project_f64(int n, int sh_degree, const double* means, const double* log_scales, const double* quats,
                    const double* logits, const double* sh, const double* cam, int W, int H, double* means2d,
                    double* conics, double* depths, int32_t* radii, double* opac, double* colors,
                    int32_t* rects, uint32_t* tiles, double* cov2d, int32_t* radius_3dgs) {
  return project_impl<double>(n, sh_degree, means, log_scales, quats, logits, sh, cam, W, H, means2d, conics,
                              depths, radii, opac, colors, rects, tiles, cov2d, radius_3dgs);
}

// -- binning: brute-force enumeration, std::stable_sort on the 64-bit key, linear range scan -------
// keys[p] = (ty * tiles_x + tx) << 32 | float_bits(depth); ids[p] = Gaussian id; Gaussians are
// enumerated in id order and each rectangle row-major (with tight 1 only the tiles tight_span
// keeps), so stability leaves equal keys in id order.
// ranges[t] = [start, end) into the sorted list; empty tiles are (0, 0). Returns the pair count.
int64_t orc_bin(int n, const uint32_t* tiles, const int32_t* rects, const float* depths, const float* means2d,
                const float* conics, const float* opac, int tight, int tiles_x, int tiles_y, int64_t capacity,
                uint64_t* keys, uint32_t* ids, uint32_t* ranges) {
  int64_t P = 0;
  for (int g = 0; g < n; ++g) P += tiles[g];
  if (P > capacity) return P;
  std::vector<std::pair<uint64_t, uint32_t>> pairs;
  pairs.reserve((size_t)P);
  for (int g = 0; g < n; ++g) {
    if (tiles[g] == 0) continue;
    uint32_t dbits;
    std::memcpy(&dbits, &depths[g], 4);
    std::vector<int32_t> span;
    if (tight)
      tight_span<float>(means2d[2 * g], means2d[2 * g + 1], conics[3 * g], conics[3 * g + 1], conics[3 * g + 2],
                        opac[g], rects + 4 * g, span);
    for (int ty = rects[4 * g + 1]; ty < rects[4 * g + 3]; ++ty)
      for (int tx = rects[4 * g + 0]; tx < rects[4 * g + 2]; ++tx) {
        if (tight && !(tx >= span[2 * (ty - rects[4 * g + 1])] && tx < span[2 * (ty - rects[4 * g + 1]) + 1]))
          continue;
        uint64_t tile = (uint64_t)ty * (uint64_t)tiles_x + (uint64_t)tx;
        pairs.push_back({(tile << 32) | (uint64_t)dbits, (uint32_t)g});
      }
  }
  std::stable_sort(pairs.begin(), pairs.end(),
                   [](const std::pair<uint64_t, uint32_t>& a, const std::pair<uint64_t, uint32_t>& b) {
                     return a.first < b.first;
                   });
  const int ntiles = tiles_x * tiles_y;
  for (int t = 0; t < 2 * ntiles; ++t) ranges[t] = 0;
  for (int64_t i = 0; i < P; ++i) {
    keys[i] = pairs[i].first;
    ids[i] = pairs[i].second;
    uint32_t t = (uint32_t)(pairs[i].first >> 32);
    if (i == 0 || (uint32_t)(pairs[i - 1].first >> 32) != t) ranges[2 * t] = (uint32_t)i;
    if (i == P - 1 || (uint32_t)(pairs[i + 1].first >> 32) != t) ranges[2 * t + 1] = (uint32_t)(i + 1);
  }
  return P;
}

// -- dense render ----------------------------------------------------------------------------------
int orc_render_f32(int n, const float* means2d, const float* conics, const float* opac, const float* colors,
                   const float* depths, const uint32_t* tiles, const int32_t* rects, int tight, int W, int H,
                   const float* bg, int64_t npix, const int32_t* pix, double band_eps, double* image,
                   double* final_T, int32_t* last_id, int32_t* n_contrib, uint8_t* fragile, int64_t* escapes,
                   int64_t* n_eval, double* depth_img) {
  return render_impl<float>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, W, H, bg, npix, pix,
                            band_eps, image, final_T, last_id, n_contrib, fragile, escapes, n_eval, depth_img);
}
int orc_render_f64(int n, const double* means2d, const double* conics, const double* opac,
                   const double* colors, const double* depths, const uint32_t* tiles, const int32_t* rects,
                   int tight, int W, int H, const double* bg, int64_t npix, const int32_t* pix, double band_eps,
                   double* image, double* final_T, int32_t* last_id, int32_t* n_contrib, uint8_t* fragile,
                   int64_t* escapes, int64_t* n_eval, double* depth_img) {
  return render_impl<double>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, W, H, bg, npix, pix,
                             band_eps, image, final_T, last_id, n_contrib, fragile, escapes, n_eval, depth_img);
}

int orc_render_bwd_f32(int n, const float* means2d, const float* conics, const float* opac, const float* colors,
                       const float* depths, const uint32_t* tiles, const int32_t* rects, int tight, int W,
                       int H, const float* bg, int64_t npix, const int32_t* pix, double band_eps,
                       const double* dL_dimg, const double* dL_ddepth, double* g2d, double* aref,
                       double* aref_plain, double* aref_terms) {
  return render_bwd_impl<float>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, W, H, bg, npix, pix,
                                band_eps, dL_dimg, dL_ddepth, g2d, aref, aref_plain, aref_terms);
}
int orc_render_bwd_f64(int n, const double* means2d, const double* conics, const double* opac,
                       const double* colors, const double* depths, const uint32_t* tiles, const int32_t* rects,
                       int tight, int W, int H, const double* bg, int64_t npix, const int32_t* pix, double band_eps,
                       const double* dL_dimg, const double* dL_ddepth, double* g2d, double* aref,
                       double* aref_plain, double* aref_terms) {
  return render_bwd_impl<double>(n, means2d, conics, opac, colors, depths, tiles, rects, tight, W, H, bg, npix, pix,
                                 band_eps, dL_dimg, dL_ddepth, g2d, aref, aref_plain, aref_terms);
}

int orc_project_bwd_f32(int n, int sh_degree, const float* means, const float* log_scales, const float* quats,
                        const float* logits, const float* sh, const float* cam, int W, int H, const double* g2d,
                        const double* aref2d, double* d_means, double* d_log_scales, double* d_quats,
                        double* d_logits, double* d_sh, double* aref_raw) {
  return project_bwd_impl<float>(n, sh_degree, means, log_scales, quats, logits, sh, cam, W, H, g2d, aref2d,
                                 d_means, d_log_scales, d_quats, d_logits, d_sh, aref_raw);
}
int orc_project_bwd_f64(int n, int sh_degree, const double* means, const double* log_scales,
                        const double* quats, const double* logits, const double* sh, const double* cam, int W,
                        int H, const double* g2d, const double* aref2d, double* d_means, double* d_log_scales,
                        double* d_quats, double* d_logits, double* d_sh, double* aref_raw) {
  return project_bwd_impl<double>(n, sh_degree, means, log_scales, quats, logits, sh, cam, W, H, g2d, aref2d,
                                  d_means, d_log_scales, d_quats, d_logits, d_sh, aref_raw);
}

int orc_num_threads(void) { return nthreads(); }

// Thread count of the later parallel regions (timing the oracle on one core or all of them).
void orc_set_num_threads(int k) {
#ifdef _OPENMP
  if (k > 0) omp_set_num_threads(k);
#else
  (void)k;
#endif
}

}  // extern "C"
