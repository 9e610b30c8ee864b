// Row-norm kernels: LayerNorm (+adaLN modulate or +affine) fp32 -> bf16, and
// in-place q/k RMSNorm over the full width fused with the 3-D rotary.
// One workgroup per row, each thread owning 8 consecutive columns (two float4
// or one 16-byte bf16 chunk), so a 1280-token slice launches 1280 workgroups
// and every load is in flight at once; block reductions go through LDS.
// Both kernels are HBM/L2-bound.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

// sum of v over the waves [w0, w0 + nw) of the workgroup (all threads get it)
__device__ __forceinline__ float group_sum(float v, float* red, int w0, int nw) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < nw; ++w) s += red[w0 + w];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(256) void layernorm_kernel(
    float* __restrict__ x, bf16_t* __restrict__ out, int rows, int D, int rows_per_lane, float eps,
    const float* __restrict__ tab_shift, const float* __restrict__ tab_scale,
    const float* __restrict__ e_shift, const float* __restrict__ e_scale, int e_stride,
    const float* __restrict__ g, const float* __restrict__ b, PendingRes pend, uint8_t* __restrict__ out_q,
    uint16_t* __restrict__ q_scale) {
  __shared__ float red[8];
  const int row = wg_x();
  const int c = threadIdx.x * 8;
  const bool on = c < D;
  float* xr = x + (int64_t)row * D + c;
  float v[8];
  if (on) {
    f32x4 a0 = reinterpret_cast<const f32x4*>(xr)[0];
    f32x4 a1 = reinterpret_cast<const f32x4*>(xr)[1];
    if (pend.part) {  // finish the residual update of x first, and store it
      a0 = apply_pending(pend, a0, row, c, rows, D);
      a1 = apply_pending(pend, a1, row, c + 4, rows, D);
      reinterpret_cast<f32x4*>(xr)[0] = a0;
      reinterpret_cast<f32x4*>(xr)[1] = a1;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a0[e]; v[e + 4] = a1[e]; }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  const int nw = blockDim.x >> 6;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += v[e];
  const float mean = group_sum(s, red, 0, nw) / (float)D;
  float q = 0.f;
  if (on) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q += (v[e] - mean) * (v[e] - mean);
  }
  const float rstd = rsqrtf(group_sum(q, red, 0, nw) / (float)D + eps);
  if (!on) return;
  float mul[8], add[8];
  if (g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { mul[e] = g[c + e]; add[e] = b[c + e]; }
  } else {
    const int ln = row / rows_per_lane;
    const float* es = e_scale + (int64_t)ln * e_stride;
    const float* eh = e_shift + (int64_t)ln * e_stride;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mul[e] = 1.f + tab_scale[c + e] + es[c + e];
      add[e] = tab_shift[c + e] + eh[c + e];
    }
  }
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (v[e] - mean) * rstd * mul[e] + add[e];
  if (out_q) {
    // MX-FP8: a 32-column block is 4 consecutive threads (D is a multiple of 64)
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int ex = mx_shared_exp(amax);
    *reinterpret_cast<u32x2*>(out_q + (int64_t)row * D + c) = pack8_e4m3(y, mx_inv_scale(ex));
    if ((threadIdx.x & 3) == 0)
      reinterpret_cast<uint8_t*>(q_scale)[((int64_t)(c / 64) * rows + row) * 2 + ((c / 32) & 1)] =
          (uint8_t)(ex + 127);
    return;
  }
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack2bf(y[2 * e], y[2 * e + 1]);
  *reinterpret_cast<u32x4*>(out + (int64_t)row * D + c) = w;
}

// nparts groups of threads, one per part of the row (q, then k); each thread
// owns one 8-element chunk; pair j of a head is (dims 2j, 2j+1).
__global__ __launch_bounds__(512) void rmsnorm_rope_kernel(
    bf16_t* __restrict__ p, int ld, int D, int tpp, const float* __restrict__ g0,
    const float* __restrict__ g1, const float* __restrict__ cos_t, const float* __restrict__ sin_t,
    int rows_per_lane, int head_dim, float eps, uint8_t* __restrict__ out_q, uint8_t* __restrict__ q_scale,
    int ldq, const BatchEntry* __restrict__ tab, int tab_rows) {
  __shared__ float red[8];
  const int row = wg_x();
  const int part = threadIdx.x / tpp, tp = threadIdx.x % tpp;
  const int c = tp * 8;
  const bool on = c < D;
  bf16_t* pr = p + (int64_t)row * ld + part * D + c;
  u16x8 raw;
  if (on) raw = *reinterpret_cast<const u16x8*>(pr);
  // the rotary pairs' cos and sin, fetched with the row so their latency hides under the reduction
  const int half = head_dim >> 1;
  f32x4 cs = {1.f, 1.f, 1.f, 1.f}, sn = {0.f, 0.f, 0.f, 0.f};
  if (cos_t && on) {
    const int64_t t0 = (int64_t)(row % rows_per_lane) * half + ((c % head_dim) >> 1);
    cs = *reinterpret_cast<const f32x4*>(cos_t + t0);
    sn = *reinterpret_cast<const f32x4*>(sin_t + t0);
  }
  float y[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y[e] = on ? bf2f(raw[e]) : 0.f;
    ss += y[e] * y[e];
  }
  const int wpp = tpp >> 6;
  // reduce per part: waves [part * wpp, (part + 1) * wpp)
  const float tot = group_sum(ss, red, part * wpp, wpp);
  if (!on) return;
  const float rs = rsqrtf(tot / (float)D + eps);
  const float* g = tab ? tab[row / tab_rows].g : part ? g1 : g0;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] *= rs * g[c + e];
  if (cos_t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = y[2 * e], bb = y[2 * e + 1];
      y[2 * e] = a * cs[e] - bb * sn[e];
      y[2 * e + 1] = a * sn[e] + bb * cs[e];
    }
  }
  if (out_q) {
    // MX-FP8 along the row: a 32-column block is 4 consecutive threads (lanes)
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int ex = mx_shared_exp(amax);
    const int col = part * D + c;
    *reinterpret_cast<u32x2*>(out_q + (int64_t)row * ldq + col) = pack8_e4m3(y, mx_inv_scale(ex));
    if ((tp & 3) == 0) q_scale[(int64_t)row * (ldq / 32) + col / 32] = (uint8_t)(ex + 127);
    return;
  }
  u16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f2bf(y[e]);
  *reinterpret_cast<u16x8*>(pr) = o;
}

int threads_for(int D) { return ((D / 8 + 63) / 64) * 64; }

}  // namespace

hipError_t layernorm_bf16(float* x, bf16_t* out, int rows, int D, int rows_per_lane, float eps,
                          const float* tab_shift, const float* tab_scale, const float* e_shift,
                          const float* e_scale, int e_stride, const float* g, const float* b,
                          const PendingRes* pend, hipStream_t s, uint8_t* out_q, uint16_t* q_scale) {
  if (rows <= 0) return hipSuccess;
  if (D % 8 || threads_for(D) > 256) return hipErrorInvalidValue;
  if (out_q && (D % 64 || !q_scale)) return hipErrorInvalidValue;
  PendingRes p;
  if (pend && pend->part) {
    if (pend->nparts < 1 || !pend->bias || (pend->gate_tab && pend->rows_per_lane <= 0))
      return hipErrorInvalidValue;
    p = *pend;
  }
  launch_timed(layernorm_kernel, rows, threads_for(D), s, x, out, rows, D, rows_per_lane, eps, tab_shift, tab_scale,
               e_shift, e_scale, e_stride, g, b, p, out_q, q_scale);
  return hipGetLastError();
}

hipError_t rmsnorm_rope_bf16(bf16_t* p, int ld, int rows, int D, int nparts, const float* g0,
                             const float* g1, const float* cos_t, const float* sin_t,
                             int rows_per_lane, int head_dim, float eps, hipStream_t s, uint8_t* out_q,
                             uint8_t* q_scale, int ldq) {
  if (rows <= 0) return hipSuccess;
  const int tpp = threads_for(D);
  if (D % 8 || ld % 8 || head_dim % 8 || nparts < 1 || nparts > 2 || tpp * nparts > 512)
    return hipErrorInvalidValue;
  if (out_q && (D % 32 || !q_scale || ldq % 32 || ldq < nparts * D)) return hipErrorInvalidValue;
  launch_timed(rmsnorm_rope_kernel, rows, tpp * nparts, s, p, ld, D, tpp, g0, g1, cos_t, sin_t, rows_per_lane,
               head_dim, eps, out_q, q_scale, ldq, nullptr, 1);
  return hipGetLastError();
}

hipError_t rmsnorm_bf16_table(bf16_t* p, int ld, int rows, int D, const BatchEntry* tab, int rows_per_entry,
                              float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int tpp = threads_for(D);
  if (D % 8 || ld % 8 || ld < D || tpp > 512 || !tab || rows_per_entry <= 0) return hipErrorInvalidValue;
  launch_timed(rmsnorm_rope_kernel, rows, tpp, s, p, ld, D, tpp, nullptr, nullptr, nullptr, nullptr, 1, 8, eps, nullptr,
               nullptr, 0, tab, rows_per_entry);
  return hipGetLastError();
}

hipError_t set_wg_reverse_norm(int r) { return set_wg_reverse(r); }

}  // namespace fh
