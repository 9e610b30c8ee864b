// Float32 debug path (FH_PREC_FP32): every activation and every product in
// float32, the bf16 weights widened exactly. Plain, unfused-where-it-matters
// kernels whose only purpose is a tight check of the block structure against
// the float64 oracle; the bf16 path's tiled MFMA kernels are the product.
#include <hip/hip_runtime.h>

#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int T = 64;        // GEMM tile (rows and columns)
constexpr int KB = 16;       // GEMM K step
constexpr int MAXKEYS = 4096;

// precise tanh-GELU: 0.5 z (1 + tanh(u)) = z / (1 + exp(-2u)), u = sqrt(2/pi)(z + 0.044715 z^3)
__device__ __forceinline__ float gelu_precise(float z) {
  const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  return z / (1.0f + expf(-2.0f * u));
}

// sum (or max) over a workgroup of NW waves; every thread gets the result
template <int NW, bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
  v = MAX ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // red may still be read by a previous reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// C[M, N] = A[M, K] (f32) W[N, K]^T (bf16) in float32, 64 x 64 tiles, 4 x 4
// results per thread, K in order; epilogues as EpiF32.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const bf16_t* __restrict__ W, int ldw, int M, int N,
                                                       int K, EpiF32Args ep) {
  __shared__ float As[KB][T + 4];
  __shared__ float Ws[KB][T + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row lr of the tile, 4 values from column lk
  const float* ap = A + (int64_t)min(m0 + lr, M - 1) * lda + lk;
  const bf16_t* wp = W + (int64_t)(n0 + lr) * ldw + lk;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KB) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(ap + k0);
    const u32x2 w = *reinterpret_cast<const u32x2*>(wp + k0);
#pragma unroll
    for (int e = 0; e < 4; ++e) As[lk + e][lr] = a[e];
    Ws[lk + 0][lr] = bf2f((bf16_t)(w.x & 0xffffu));
    Ws[lk + 1][lr] = bf2f((bf16_t)(w.x >> 16));
    Ws[lk + 2][lr] = bf2f((bf16_t)(w.y & 0xffffu));
    Ws[lk + 3][lr] = bf2f((bf16_t)(w.y >> 16));
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float av[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      const float v = acc[i][j] + ep.bias[n];
      if (EPI == F32_OUT) {
        ep.out[(int64_t)m * ep.ldo + n] = v;
      } else if (EPI == F32_GELU) {
        ep.out[(int64_t)m * ep.ldo + n] = gelu_precise(v);
      } else if (EPI == F32_RES) {
        ep.x[(int64_t)m * ep.ldx + n] += v;
      } else {
        const float g = ep.gate_tab[n] + ep.gate_e0[(int64_t)(m / ep.rows_per_lane) * ep.gate_stride + n];
        ep.x[(int64_t)m * ep.ldx + n] += g * v;
      }
    }
  }
}

// one 256-thread workgroup per row; two passes (mean, then centred variance)
__global__ __launch_bounds__(256) void layernorm_f32_kernel(const float* __restrict__ x, float* __restrict__ out,
                                                            int D, int rows_per_lane, float eps,
                                                            const float* __restrict__ tab_shift,
                                                            const float* __restrict__ tab_scale,
                                                            const float* __restrict__ e_shift,
                                                            const float* __restrict__ e_scale, int e_stride,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ b) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const float* xr = x + (int64_t)row * D;
  float s = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) s += xr[c];
  const float mean = block_reduce<4, false>(s, red) / (float)D;
  float v = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float d = xr[c] - mean;
    v = fmaf(d, d, v);
  }
  const float var = block_reduce<4, false>(v, red) / (float)D;
  const float rs = 1.0f / sqrtf(var + eps);
  const int lane_row = row / rows_per_lane;
  float* orow = out + (int64_t)row * D;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float n = (xr[c] - mean) * rs;
    float y;
    if (g) {
      y = n * g[c] + b[c];
    } else {
      const float sc = tab_scale[c] + e_scale[(int64_t)lane_row * e_stride + c];
      const float sh = tab_shift[c] + e_shift[(int64_t)lane_row * e_stride + c];
      y = n * (1.0f + sc) + sh;
    }
    orow[c] = y;
  }
}

// in-place RMSNorm of one row (first D columns, gain g), then optionally the
// pairwise rotation: pair j of a head (columns 2j, 2j+1 within the head) by
// angle table row (row mod rows_per_lane), column j
__global__ __launch_bounds__(256) void rmsnorm_rope_f32_kernel(float* __restrict__ p, int ld, int D,
                                                               const float* __restrict__ g,
                                                               const float* __restrict__ cos_t,
                                                               const float* __restrict__ sin_t,
                                                               int rows_per_lane, int head_dim, float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  float* r = p + (int64_t)row * ld;
  float s = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) s = fmaf(r[c], r[c], s);
  const float ms = block_reduce<4, false>(s, red) / (float)D;
  const float rs = 1.0f / sqrtf(ms + eps);
  const int half = head_dim / 2;
  const int tok = row % rows_per_lane;
  for (int q = threadIdx.x; q < D / 2; q += 256) {
    const int c = 2 * q;
    const float a = r[c] * rs * g[c];
    const float bb = r[c + 1] * rs * g[c + 1];
    if (cos_t) {
      const int j = q % half;
      const float cs = cos_t[(int64_t)tok * half + j], sn = sin_t[(int64_t)tok * half + j];
      r[c] = a * cs - bb * sn;
      r[c + 1] = a * sn + bb * cs;
    } else {
      r[c] = a;
      r[c + 1] = bb;
    }
  }
}

// Exact softmax attention of one query row and head (128 threads = head_dim):
// the scores of its key range in LDS, max-subtracted exponentials, then the
// weighted sum of value rows. Key range: all Nk keys of the lane, or (local)
// the apf keys of the query's latent frame (row / hw).
__global__ __launch_bounds__(128) void attn_f32_kernel(const float* __restrict__ q, int ldq,
                                                       const float* __restrict__ k, int ldk,
                                                       const float* __restrict__ v, int ldv, float* __restrict__ o,
                                                       int ldo, int Nq, int Nk, float scale, int hw, int apf,
                                                       int local) {
  __shared__ float qs[128];
  __shared__ float sc[MAXKEYS];
  __shared__ float red[2];
  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t qrow = (int64_t)b * Nq + n;
  qs[t] = q[qrow * ldq + h * 128 + t];
  const int lo = local ? (n / hw) * apf : 0;
  const int hi = local ? lo + apf : Nk;
  __syncthreads();
  float mx = -INFINITY;
  for (int j = lo + t; j < hi; j += 128) {
    const float* kr = k + ((int64_t)b * Nk + j) * ldk + h * 128;
    float d = 0.f;
    for (int e = 0; e < 128; ++e) d = fmaf(qs[e], kr[e], d);
    d *= scale;
    sc[j - lo] = d;
    mx = fmaxf(mx, d);
  }
  mx = block_reduce<2, true>(mx, red);
  float sum = 0.f;
  for (int j = lo + t; j < hi; j += 128) {
    const float e = expf(sc[j - lo] - mx);
    sc[j - lo] = e;
    sum += e;
  }
  sum = block_reduce<2, false>(sum, red);  // also orders the writes of sc before the reads below
  float acc = 0.f;
  for (int j = lo; j < hi; ++j) acc = fmaf(sc[j - lo], v[((int64_t)b * Nk + j) * ldv + h * 128 + t], acc);
  o[qrow * ldo + h * 128 + t] = acc / sum;
}

}  // namespace

hipError_t gemm_f32(int epi, const float* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                    const EpiF32Args& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % T || K % KB || lda % 4 || ldw % 4 || !ep.bias) return hipErrorInvalidValue;
  if ((epi == F32_OUT || epi == F32_GELU) && !ep.out) return hipErrorInvalidValue;
  if ((epi == F32_RES || epi == F32_GATED_RES) && !ep.x) return hipErrorInvalidValue;
  if (epi == F32_GATED_RES && (!ep.gate_tab || !ep.gate_e0 || ep.rows_per_lane <= 0)) return hipErrorInvalidValue;
  const dim3 grid(N / T, (M + T - 1) / T), block(256);
  switch (epi) {
    case F32_OUT: launch_timed(gemm_f32_kernel<F32_OUT>, grid, block, s, A, lda, W, ldw, M, N, K, ep); break;
    case F32_GELU: launch_timed(gemm_f32_kernel<F32_GELU>, grid, block, s, A, lda, W, ldw, M, N, K, ep); break;
    case F32_RES: launch_timed(gemm_f32_kernel<F32_RES>, grid, block, s, A, lda, W, ldw, M, N, K, ep); break;
    case F32_GATED_RES: launch_timed(gemm_f32_kernel<F32_GATED_RES>, grid, block, s, A, lda, W, ldw, M, N, K, ep); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t layernorm_f32(const float* x, float* out, int rows, int D, int rows_per_lane, float eps,
                         const float* tab_shift, const float* tab_scale, const float* e_shift,
                         const float* e_scale, int e_stride, const float* g, const float* b, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D <= 0 || rows_per_lane <= 0 || (!g && (!tab_shift || !tab_scale || !e_shift || !e_scale)) ||
      (g && !b))
    return hipErrorInvalidValue;
  launch_timed(layernorm_f32_kernel, rows, 256, s, x, out, D, rows_per_lane, eps, tab_shift, tab_scale, e_shift,
               e_scale, e_stride, g, b);
  return hipGetLastError();
}

hipError_t rmsnorm_rope_f32(float* p, int ld, int rows, int D, const float* g, const float* cos_t,
                            const float* sin_t, int rows_per_lane, int head_dim, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D % 2 || !g || rows_per_lane <= 0 || head_dim % 2 || (cos_t && D % head_dim)) return hipErrorInvalidValue;
  launch_timed(rmsnorm_rope_f32_kernel, rows, 256, s, p, ld, D, g, cos_t, sin_t, rows_per_lane, head_dim, eps);
  return hipGetLastError();
}

hipError_t attn_f32(const float* q, int ldq, const float* k, int ldk, const float* v, int ldv, float* o,
                    int ldo, int B, int Nq, int Nk, int n_heads, float scale, int hw, int apf, int local,
                    hipStream_t s) {
  if (B <= 0 || Nq <= 0) return hipSuccess;
  if (Nk <= 0 || n_heads <= 0 || n_heads > 65535 || B > 65535) return hipErrorInvalidValue;
  if (local ? (apf <= 0 || apf > MAXKEYS || hw <= 0 || (int64_t)((Nq - 1) / hw + 1) * apf > Nk) : Nk > MAXKEYS)
    return hipErrorInvalidValue;
  launch_timed(attn_f32_kernel, dim3(Nq, n_heads, B), 128, s, q, ldq, k, ldk, v, ldv, o, ldo, Nq, Nk, scale, hw, apf,
               local);
  return hipGetLastError();
}

}  // namespace fh
