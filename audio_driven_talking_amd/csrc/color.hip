// Colour correction after the VAE decode: each decoded frame's colours are
// moved to the reference picture's CIELAB statistics (gizai:flashhead
// reference page, overview paragraph: Lab means and deviations; audio-cpp
// page "SoulX-FlashHead", section Generate: a strength, 1 by default, 0
// disabling it; section Variant boundaries: colour processing on the device
// in F32).
//
// sRGB in [0, 1] -> linear (the sRGB curve) -> XYZ (BT.709 primaries, D65 at
// the sRGB chromaticity 0.3127, 0.3290) -> CIELAB relative to that white.
// Per frame and Lab channel: v' = mu_ref + (v - mu) sd_ref / sd (mu_ref where
// sd = 0), blended v + s (v' - v), back to sRGB, clamped to [0, 1].
//
// Layout: RGB planes, frames [3][F][H*W] and picture [3][H'*W'], float32.
// Three kernels: per-chunk channel sums of shifted Lab and its square in
// float64 (every image: the frames and the picture), a per-frame reduction of
// the chunks in index order to the transfer coefficients, and the per-pixel
// transfer in float32. The frames are read twice and written once; the sRGB
// curve's powers dominate the arithmetic.
#include <mutex>

#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int CM_CHUNK = 2048;  // pixels per statistics workgroup (8 per thread)

// sRGB -> XYZ for BT.709 primaries and the D65 white (0.3127, 0.3290), with
// the white folded in: m maps linear RGB to (X/Xn, Y/Yn, Z/Zn), minv maps
// (X/Xn, Y/Yn, Z/Zn) back to linear RGB. Formed from the chromaticities on
// the host in float64.
struct ColorTables {
  float m[9];
  float minv[9];
};

// x^e for x > 0 as 2^(e log2 x) on the hardware log2 / exp2 (a few 1e-7
// relative on the ranges used here: x >= 0.003, |e log2 x| < 20)
__device__ __forceinline__ float pow_pos(float x, float e) {
  return __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(x));
}
__device__ __forceinline__ float srgb_to_lin(float c) {
  return c <= 0.04045f ? c * (1.0f / 12.92f) : pow_pos((c + 0.055f) * (1.0f / 1.055f), 2.4f);
}
__device__ __forceinline__ float lin_to_srgb(float c) {
  return c <= 0.0031308f ? 12.92f * c : 1.055f * pow_pos(c, 1.0f / 2.4f) - 0.055f;
}
// CIELAB's f and its inverse (delta = 6/29)
__device__ __forceinline__ float lab_f(float t) {
  constexpr float d = 6.0f / 29.0f;
  return t > d * d * d ? pow_pos(t, 1.0f / 3.0f) : t * (1.0f / (3.0f * d * d)) + 4.0f / 29.0f;
}
__device__ __forceinline__ float lab_finv(float t) {
  constexpr float d = 6.0f / 29.0f;
  return t > d ? t * t * t : 3.0f * d * d * (t - 4.0f / 29.0f);
}

__device__ __forceinline__ void rgb_to_lab(const ColorTables& T, const float rgb[3], float lab[3]) {
  const float r = srgb_to_lin(rgb[0]), g = srgb_to_lin(rgb[1]), b = srgb_to_lin(rgb[2]);
  const float fx = lab_f(T.m[0] * r + T.m[1] * g + T.m[2] * b);
  const float fy = lab_f(T.m[3] * r + T.m[4] * g + T.m[5] * b);
  const float fz = lab_f(T.m[6] * r + T.m[7] * g + T.m[8] * b);
  lab[0] = 116.0f * fy - 16.0f;
  lab[1] = 500.0f * (fx - fy);
  lab[2] = 200.0f * (fy - fz);
}

__device__ __forceinline__ void lab_to_rgb(const ColorTables& T, const float lab[3], float rgb[3]) {
  const float fy = (lab[0] + 16.0f) * (1.0f / 116.0f);
  const float x = lab_finv(fy + lab[1] * (1.0f / 500.0f));
  const float y = lab_finv(fy);
  const float z = lab_finv(fy - lab[2] * (1.0f / 200.0f));
#pragma unroll
  for (int i = 0; i < 3; ++i)
    rgb[i] = fminf(fmaxf(lin_to_srgb(T.minv[3 * i] * x + T.minv[3 * i + 1] * y + T.minv[3 * i + 2] * z), 0.0f), 1.0f);
}

// Pixel group g (4 consecutive pixels when VEC) of the planar image at
// `base` with plane stride `ps` and n pixels: rgb[c][j].
template <bool VEC>
__device__ __forceinline__ int load_px(const float* base, int64_t ps, int64_t n, int64_t p0, float rgb[3][4]) {
  if (VEC && p0 + 3 < n) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(base + c * ps + p0);
      rgb[c][0] = v.x, rgb[c][1] = v.y, rgb[c][2] = v.z, rgb[c][3] = v.w;
    }
    return 4;
  }
  const int m = VEC ? (int)(n - p0 < 4 ? n - p0 : 4) : 1;
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < 3; ++c) rgb[c][j] = j < m ? base[c * ps + p0 + j] : 0.0f;
  return m;
}

// partial[img][chunk][6]: sums of d and d^2 per Lab channel over the chunk's
// pixels, with d = Lab - Lab(first pixel of the image) (shifted sums: exact
// zeros for a flat image, little cancellation otherwise). Images 0 .. F-1
// are the frames (planes [3][F][HW]), image F the picture ([3][HW']);
// chunks past an image's end add zeros.
template <bool VEC>
__global__ __launch_bounds__(256) void color_stats_kernel(const float* __restrict__ frames, int64_t npix,
                                                          const float* __restrict__ pic, int64_t npix_ref,
                                                          int F, ColorTables T, double* __restrict__ partial) {
  __shared__ double red[6][256];
  const int img = blockIdx.y, chunk = wg_x();
  const bool is_ref = img == F;
  const float* base = is_ref ? pic : frames + (int64_t)img * npix;
  const int64_t ps = is_ref ? npix_ref : (int64_t)F * npix;
  const int64_t n = is_ref ? npix_ref : npix;
  float k[3];
  {
    const float rgb0[3] = {base[0], base[ps], base[2 * ps]};
    rgb_to_lab(T, rgb0, k);
  }
  // a thread's 8 pixels are summed in float32 (|d| <= 100: a few 1e-5 at
  // most), the threads' and chunks' sums in float64
  float acc[6] = {0, 0, 0, 0, 0, 0};
  auto add = [&](const float px[3]) {
    float lab[3];
    rgb_to_lab(T, px, lab);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const float d = lab[c] - k[c];
      acc[c] += d;
      acc[3 + c] += d * d;
    }
  };
  if (VEC) {
    // 8 consecutive pixels per thread, all six float4 loads issued before any
    // arithmetic; n % 4 == 0, so each half is whole or absent
    const int64_t p0 = (int64_t)chunk * CM_CHUNK + (int64_t)threadIdx.x * 8;
    float4 v[2][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 3; ++c)
        v[h][c] = p0 + 4 * h < n ? *reinterpret_cast<const float4*>(base + c * ps + p0 + 4 * h) : make_float4(0, 0, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (p0 + 4 * h < n) {
        const float q[3][4] = {{v[h][0].x, v[h][0].y, v[h][0].z, v[h][0].w},
                               {v[h][1].x, v[h][1].y, v[h][1].z, v[h][1].w},
                               {v[h][2].x, v[h][2].y, v[h][2].z, v[h][2].w}};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float px[3] = {q[0][j], q[1][j], q[2][j]};
          add(px);
        }
      }
  } else {
    for (int i = 0; i < CM_CHUNK / 256; ++i) {
      const int64_t p = (int64_t)chunk * CM_CHUNK + i * 256 + threadIdx.x;
      if (p < n) {
        const float px[3] = {base[p], base[ps + p], base[2 * ps + p]};
        add(px);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 6; ++c) red[c][threadIdx.x] = (double)acc[c];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {  // pairwise tree, the same order every time
    if (threadIdx.x < s)
#pragma unroll
      for (int c = 0; c < 6; ++c) red[c][threadIdx.x] += red[c][threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x < 6) partial[((int64_t)img * gridDim.x + chunk) * 6 + threadIdx.x] = red[threadIdx.x][0];
}

// Mean and population deviation of image img from its partials: thread t adds
// chunks t, t + 256, ... in order, then a pairwise tree over the threads
// (a fixed order). Needs blockDim.x == 256; every thread gets the result.
__device__ void image_stats(const double* partial, int nchunks, int img, int64_t n, const float k[3], double mu[3],
                            double sd[3], double (*red)[256]) {
  double s[6] = {0, 0, 0, 0, 0, 0};
  for (int q = threadIdx.x; q < nchunks; q += 256)
#pragma unroll
    for (int c = 0; c < 6; ++c) s[c] += partial[((int64_t)img * nchunks + q) * 6 + c];
#pragma unroll
  for (int c = 0; c < 6; ++c) red[c][threadIdx.x] = s[c];
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h)
#pragma unroll
      for (int c = 0; c < 6; ++c) red[c][threadIdx.x] += red[c][threadIdx.x + h];
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const double m = red[c][0] / (double)n;
    mu[c] = (double)k[c] + m;
    sd[c] = sqrt(fmax(red[3 + c][0] / (double)n - m * m, 0.0));
  }
  __syncthreads();  // red is reused
}

// A channel whose deviation is below this many Lab units counts as flat: on
// a grey frame a* and b* hold only rounding noise (about 1e-5 in float32),
// which sd_ref / sd would turn into arbitrary chroma.
constexpr double FLAT_SD = 1e-3;

// coef[f][9]: per Lab channel the frame's mean, the picture's mean and the
// scale sd_ref / sd (0 where sd < FLAT_SD). One workgroup of 256 per frame; each
// also reduces the picture's partials.
__global__ __launch_bounds__(256) void color_finalize_kernel(const float* __restrict__ frames, int64_t npix,
                                                             const float* __restrict__ pic, int64_t npix_ref,
                                                             const double* __restrict__ partial, int nchunks, int F,
                                                             ColorTables T, float* __restrict__ coef) {
  __shared__ double red[6][256];
  const int f = wg_x();
  const int64_t fps = (int64_t)F * npix;
  float kf[3], kr[3];
  {
    const float a[3] = {frames[(int64_t)f * npix], frames[fps + (int64_t)f * npix], frames[2 * fps + (int64_t)f * npix]};
    const float b[3] = {pic[0], pic[npix_ref], pic[2 * npix_ref]};
    rgb_to_lab(T, a, kf);
    rgb_to_lab(T, b, kr);
  }
  double mu[3], sd[3], mur[3], sdr[3];
  image_stats(partial, nchunks, f, npix, kf, mu, sd, red);
  image_stats(partial, nchunks, F, npix_ref, kr, mur, sdr, red);
  if (threadIdx.x == 0)
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      coef[f * 9 + c] = (float)mu[c];
      coef[f * 9 + 3 + c] = (float)mur[c];
      coef[f * 9 + 6 + c] = sd[c] >= FLAT_SD ? (float)(sdr[c] / sd[c]) : 0.0f;
    }
}

// One thread per pixel group: Lab, moved toward the picture's statistics by
// `strength`, back to sRGB, clamped. frames and out may be the same buffer
// (each element is read, then written, by one thread).
template <bool VEC>
__global__ __launch_bounds__(256) void color_apply_kernel(const float* frames, int64_t npix, int F,
                                                          const float* __restrict__ coef, float strength,
                                                          ColorTables T, float* out) {
  constexpr int PX = VEC ? 4 : 1;
  const int64_t groups_per_frame = (npix + PX - 1) / PX;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)F * groups_per_frame) return;
  const int f = (int)(g / groups_per_frame);
  const int64_t p0 = (g - (int64_t)f * groups_per_frame) * PX;
  const int64_t ps = (int64_t)F * npix;
  const float* src = frames + (int64_t)f * npix;
  float* dst = out + (int64_t)f * npix;
  const float* cf = coef + f * 9;
  float rgb[3][4];
  const int m = load_px<VEC>(src, ps, npix, p0, rgb);
  for (int j = 0; j < m; ++j) {
    const float px[3] = {rgb[0][j], rgb[1][j], rgb[2][j]};
    float lab[3];
    rgb_to_lab(T, px, lab);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const float matched = cf[3 + c] + (lab[c] - cf[c]) * cf[6 + c];
      lab[c] += strength * (matched - lab[c]);
    }
    float o[3];
    lab_to_rgb(T, lab, o);
#pragma unroll
    for (int c = 0; c < 3; ++c) rgb[c][j] = o[c];
  }
  if (VEC && m == 4) {
#pragma unroll
    for (int c = 0; c < 3; ++c)
      *reinterpret_cast<float4*>(dst + c * ps + p0) = make_float4(rgb[c][0], rgb[c][1], rgb[c][2], rgb[c][3]);
  } else {
    for (int j = 0; j < m; ++j)
#pragma unroll
      for (int c = 0; c < 3; ++c) dst[c * ps + p0 + j] = rgb[c][j];
  }
}

// XYZ at Y = 1 of chromaticity (x, y)
void xyz_of(double x, double y, double v[3]) {
  v[0] = x / y;
  v[1] = 1.0;
  v[2] = (1.0 - x - y) / y;
}

// 3x3 inverse by the adjugate
void inv3(const double a[9], double r[9]) {
  const double det = a[0] * (a[4] * a[8] - a[5] * a[7]) - a[1] * (a[3] * a[8] - a[5] * a[6]) +
                     a[2] * (a[3] * a[7] - a[4] * a[6]);
  r[0] = (a[4] * a[8] - a[5] * a[7]) / det;
  r[1] = (a[2] * a[7] - a[1] * a[8]) / det;
  r[2] = (a[1] * a[5] - a[2] * a[4]) / det;
  r[3] = (a[5] * a[6] - a[3] * a[8]) / det;
  r[4] = (a[0] * a[8] - a[2] * a[6]) / det;
  r[5] = (a[2] * a[3] - a[0] * a[5]) / det;
  r[6] = (a[3] * a[7] - a[4] * a[6]) / det;
  r[7] = (a[1] * a[6] - a[0] * a[7]) / det;
  r[8] = (a[0] * a[4] - a[1] * a[3]) / det;
}

// the primaries' XYZ as columns, each scaled so that R = G = B = 1 is the white
ColorTables color_tables() {
  const double prim[3][2] = {{0.64, 0.33}, {0.30, 0.60}, {0.15, 0.06}};
  double P[9], w[3], Pinv[9], M[9], Minv[9];
  for (int j = 0; j < 3; ++j) {
    double v[3];
    xyz_of(prim[j][0], prim[j][1], v);
    for (int i = 0; i < 3; ++i) P[3 * i + j] = v[i];
  }
  xyz_of(0.3127, 0.3290, w);
  inv3(P, Pinv);
  for (int j = 0; j < 3; ++j) {
    const double sj = Pinv[3 * j] * w[0] + Pinv[3 * j + 1] * w[1] + Pinv[3 * j + 2] * w[2];
    for (int i = 0; i < 3; ++i) M[3 * i + j] = P[3 * i + j] * sj;
  }
  inv3(M, Minv);
  ColorTables T;
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      T.m[3 * i + j] = (float)(M[3 * i + j] / w[i]);      // rows scaled: X/Xn, Y/Yn, Z/Zn
      T.minv[3 * i + j] = (float)(Minv[3 * i + j] * w[j]);  // columns scaled back
    }
  return T;
}

int color_chunks(int64_t npix, int64_t npix_ref) {
  const int64_t n = npix > npix_ref ? npix : npix_ref;
  return (int)((n + CM_CHUNK - 1) / CM_CHUNK);
}

size_t partial_bytes(int F, int nchunks) { return ((size_t)(F + 1) * nchunks * 6 * sizeof(double) + 255) / 256 * 256; }

}  // namespace

size_t color_match_workspace(int F, int64_t npix, int64_t npix_ref) {
  return partial_bytes(F, color_chunks(npix, npix_ref)) + (size_t)F * 9 * sizeof(float);
}

// Sizes are checked by the caller: F in [1, 65534], npix and npix_ref >= 1,
// workspace of color_match_workspace bytes, 256-byte aligned.
hipError_t color_match(const float* frames, int F, int64_t npix, const float* pic, int64_t npix_ref, float strength,
                       float* out, void* ws, hipStream_t s) {
  const int nchunks = color_chunks(npix, npix_ref);
  double* partial = (double*)ws;
  float* coef = (float*)((char*)ws + partial_bytes(F, nchunks));
  const ColorTables T = color_tables();
  // float4 planes need every plane offset (multiples of npix, npix_ref) and base 16-byte aligned
  const bool vec = npix % 4 == 0 && npix_ref % 4 == 0 && ((uintptr_t)frames & 15) == 0 && ((uintptr_t)pic & 15) == 0 &&
                   ((uintptr_t)out & 15) == 0;
  const int64_t groups = vec ? (int64_t)F * (npix / 4) : (int64_t)F * npix;
  const dim3 sgrid(nchunks, F + 1);
  if (vec)
    launch_timed(color_stats_kernel<true>, sgrid, 256, s, frames, npix, pic, npix_ref, F, T, partial);
  else
    launch_timed(color_stats_kernel<false>, sgrid, 256, s, frames, npix, pic, npix_ref, F, T, partial);
  launch_timed(color_finalize_kernel, F, 256, s, frames, npix, pic, npix_ref, partial, nchunks, F, T, coef);
  const unsigned agrid = (unsigned)((groups + 255) / 256);
  if (vec)
    launch_timed(color_apply_kernel<true>, agrid, 256, s, frames, npix, F, coef, strength, T, out);
  else
    launch_timed(color_apply_kernel<false>, agrid, 256, s, frames, npix, F, coef, strength, T, out);
  return hipGetLastError();
}


// ---- statistics scratch in a static device array, for callers that cannot
// allocate (fh_color_match_noalloc). Every GPU the library runs on holds its
// own copy of the array until the process ends. In host code `scratch` names
// a host-side stand-in, not device memory: the device address of each GPU's
// copy comes from hipGetSymbolAddress, once per device, and only that address
// is ever passed to a kernel.
namespace {
constexpr size_t COLOR_SCRATCH_BYTES = (size_t)4 << 20;
static __device__ __align__(256) char scratch[COLOR_SCRATCH_BYTES];
constexpr int MAX_SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[MAX_SCRATCH_DEVICES] = {};
}  // namespace

size_t color_scratch_bytes() { return COLOR_SCRATCH_BYTES; }

hipError_t color_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t set_wg_reverse_color(int r) { return set_wg_reverse(r); }

}  // namespace fh
