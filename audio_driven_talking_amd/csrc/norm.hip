// Row-norm kernels: LayerNorm (+adaLN modulate or +affine) fp32 -> bf16, and
// in-place q/k RMSNorm over the full width fused with the 3-D rotary.
// One wave per row, 4 rows per 256-thread workgroup; the row stays in
// registers between the statistics pass and the write pass. HBM-bound.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int MAXV4 = 8;  // float4 per lane: rows up to 64*4*8 = 2048 wide

__global__ __launch_bounds__(256) void layernorm_kernel(
    const float* __restrict__ x, bf16_t* __restrict__ out, int rows, int D, int rows_per_lane,
    float eps, const float* __restrict__ tab_shift, const float* __restrict__ tab_scale,
    const float* __restrict__ e_shift, const float* __restrict__ e_scale, int e_stride,
    const float* __restrict__ g, const float* __restrict__ b) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nv = D >> 2;  // float4 chunks in the row; lane takes chunks lane + 64 i
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)row * D);
  float4 v[MAXV4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV4; ++i)
    if (i * 64 + lane < nv) {
      v[i] = xr[i * 64 + lane];
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV4; ++i)
    if (i * 64 + lane < nv) {
      float a = v[i].x - mean, bb = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + bb * bb) + (c * c + d * d);
    }
  const float rstd = rsqrtf(wave_sum(q) / (float)D + eps);
  const int ln = row / rows_per_lane;
  uint2* orow = reinterpret_cast<uint2*>(out + (int64_t)row * D);
#pragma unroll
  for (int i = 0; i < MAXV4; ++i)
    if (i * 64 + lane < nv) {
      const int col = (i * 64 + lane) * 4;
      float4 mul, add;
      if (g) {
        mul = *reinterpret_cast<const float4*>(g + col);
        add = *reinterpret_cast<const float4*>(b + col);
      } else {
        float4 ts = *reinterpret_cast<const float4*>(tab_scale + col);
        float4 th = *reinterpret_cast<const float4*>(tab_shift + col);
        float4 es = *reinterpret_cast<const float4*>(e_scale + (int64_t)ln * e_stride + col);
        float4 eh = *reinterpret_cast<const float4*>(e_shift + (int64_t)ln * e_stride + col);
        mul = make_float4(1.f + ts.x + es.x, 1.f + ts.y + es.y, 1.f + ts.z + es.z, 1.f + ts.w + es.w);
        add = make_float4(th.x + eh.x, th.y + eh.y, th.z + eh.z, th.w + eh.w);
      }
      float y0 = (v[i].x - mean) * rstd * mul.x + add.x;
      float y1 = (v[i].y - mean) * rstd * mul.y + add.y;
      float y2 = (v[i].z - mean) * rstd * mul.z + add.z;
      float y3 = (v[i].w - mean) * rstd * mul.w + add.w;
      uint2 w;
      w.x = pack2bf(y0, y1);
      w.y = pack2bf(y2, y3);
      orow[i * 64 + lane] = w;
    }
}

constexpr int MAXC8 = 4;  // 8-element chunks per lane per part: width up to 64*8*4 = 2048

__global__ __launch_bounds__(256) void rmsnorm_rope_kernel(
    bf16_t* __restrict__ p, int ld, int rows, int D, int nparts, const float* __restrict__ g0,
    const float* __restrict__ g1, const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    int rows_per_lane, int head_dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nc = D >> 3;  // 8-element chunks in the row; lane takes chunks lane + 64 i
  const int half = head_dim >> 1;
  const int tok = row % rows_per_lane;
  for (int part = 0; part < nparts; ++part) {
    u16x8* pr = reinterpret_cast<u16x8*>(p + (int64_t)row * ld + part * D);
    const float* g = part ? g1 : g0;
    u16x8 v[MAXC8];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC8; ++i)
      if (i * 64 + lane < nc) {
        v[i] = pr[i * 64 + lane];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float f = bf2f(v[i][e]);
          ss += f * f;
        }
      }
    const float rs = rsqrtf(wave_sum(ss) / (float)D + eps);
#pragma unroll
    for (int i = 0; i < MAXC8; ++i)
      if (i * 64 + lane < nc) {
        const int col = (i * 64 + lane) * 8;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = bf2f(v[i][e]) * rs * g[col + e];
        if (cos_t) {
          const int j0 = (col % head_dim) >> 1;  // first pair of this chunk within its head
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = cos_t[(int64_t)tok * half + j0 + e];
            const float s = sin_t[(int64_t)tok * half + j0 + e];
            const float a = y[2 * e], bb = y[2 * e + 1];
            y[2 * e] = a * c - bb * s;
            y[2 * e + 1] = a * s + bb * c;
          }
        }
        u16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = f2bf(y[e]);
        pr[i * 64 + lane] = o;
      }
  }
}

}  // namespace

hipError_t layernorm_bf16(const float* x, bf16_t* out, int rows, int D, int rows_per_lane, float eps,
                          const float* tab_shift, const float* tab_scale, const float* e_shift,
                          const float* e_scale, int e_stride, const float* g, const float* b,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 4 || D > 256 * MAXV4) return hipErrorInvalidValue;
  layernorm_kernel<<<(rows + 3) / 4, 256, 0, s>>>(x, out, rows, D, rows_per_lane, eps, tab_shift,
                                                  tab_scale, e_shift, e_scale, e_stride, g, b);
  return hipGetLastError();
}

hipError_t rmsnorm_rope_bf16(bf16_t* p, int ld, int rows, int D, int nparts, const float* g0,
                             const float* g1, const float* cos_t, const float* sin_t,
                             int rows_per_lane, int head_dim, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 8 || D > 512 * MAXC8 || ld % 8 || head_dim % 8) return hipErrorInvalidValue;
  rmsnorm_rope_kernel<<<(rows + 3) / 4, 256, 0, s>>>(p, ld, rows, D, nparts, g0, g1, cos_t, sin_t,
                                                     rows_per_lane, head_dim, eps);
  return hipGetLastError();
}

}  // namespace fh
