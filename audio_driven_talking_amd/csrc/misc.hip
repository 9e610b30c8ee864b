// Small kernels of the slice denoiser: rotary angle tables, timestep
// sinusoid, the time-MLP GEMVs, patch embedding, the fused output head +
// Euler update + motion pin, and conversions. All are HBM- or launch-bound.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

__global__ void rope_table_kernel(float* __restrict__ cos_t, float* __restrict__ sin_t, int F, int H,
                                  int W, int half, int nf, int nr, double theta) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_tok = (int64_t)F * H * W;
  if (i >= n_tok * half) return;
  const int tok = (int)(i / half), j = (int)(i % half);
  const int f = tok / (H * W), r = (tok / W) % H, c = tok % W;
  int pos, jl, n;
  if (j < nf) {
    pos = f; jl = j; n = nf;
  } else if (j < nf + nr) {
    pos = r; jl = j - nf; n = nr;
  } else {
    pos = c; jl = j - nf - nr; n = half - nf - nr;
  }
  const double a = (double)pos * pow(theta, -(double)jl / (double)n);
  cos_t[i] = (float)cos(a);
  sin_t[i] = (float)sin(a);
}

constexpr int MAXR = 8;
struct Times {
  float t[MAXR];
};

__global__ void sinusoid_kernel(float* __restrict__ out, Times ts, int R, int dim) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= R * dim) return;
  const int r = i / dim, k = i % dim, half = dim / 2;
  const int kk = k < half ? k : k - half;
  const double a = (double)ts.t[r] * pow(10000.0, -(double)kk / (double)half);
  out[i] = (float)(k < half ? cos(a) : sin(a));
}

// 16 outputs per 256-thread workgroup (4 per wave); the R input rows sit in LDS,
// staged in 16-byte pieces whose loads are all in flight before the first
// store (one scalar load-store round per element was the kernel's largest
// cost). A wave requests the weights of its 4 rows for a 2048-deep chunk of K
// at once (16 bytes per lane and row, 4 chunks of 512), then forms the products.
constexpr int GV_OPW = 4, GV_KC = 4;

__global__ __launch_bounds__(256) void gemv_kernel(const float* __restrict__ x, int R, int K,
                                                   const bf16_t* __restrict__ W,
                                                   const float* __restrict__ b, float* __restrict__ y,
                                                   int N, int act_in, int act_out) {
  extern __shared__ float sx[];
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    // 16-byte pieces (R K is a multiple of 8), up to 8 per thread requested
    // before the first is stored
    const int n4 = R * K / 4;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    f32x4* s4 = reinterpret_cast<f32x4*>(sx);
    for (int i0 = threadIdx.x; i0 < n4; i0 += 256 * 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 256 * u < n4) v[u] = x4[i0 + 256 * u];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 256 * u < n4) {
          f32x4 t = v[u];
          if (act_in) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = silu(t[e]);
          }
          s4[i0 + 256 * u] = t;
        }
    }
  } else {
    for (int i = threadIdx.x; i < R * K; i += 256) {
      float v = x[i];
      sx[i] = act_in ? silu(v) : v;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = wg_x() * 16 + wave * GV_OPW;
  float acc[GV_OPW][MAXR];
#pragma unroll
  for (int o = 0; o < GV_OPW; ++o)
#pragma unroll
    for (int r = 0; r < MAXR; ++r) acc[o][r] = 0.f;
  const int KC = K / 8;  // 8-element chunks per row
  for (int c0 = 0; c0 < KC; c0 += 64 * GV_KC) {
    u16x8 w[GV_OPW][GV_KC];
#pragma unroll
    for (int o = 0; o < GV_OPW; ++o)
#pragma unroll
      for (int i = 0; i < GV_KC; ++i) {
        const int kc = c0 + 64 * i + lane;
        if (n0 + o < N && kc < KC) w[o][i] = reinterpret_cast<const u16x8*>(W + (int64_t)(n0 + o) * K)[kc];
        else w[o][i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
    for (int i = 0; i < GV_KC; ++i) {
      const int kc = c0 + 64 * i + lane;
      if (kc >= KC) break;
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (r >= R) break;
        const f32x4 a = *reinterpret_cast<const f32x4*>(sx + r * K + kc * 8);
        const f32x4 c = *reinterpret_cast<const f32x4*>(sx + r * K + kc * 8 + 4);
#pragma unroll
        for (int o = 0; o < GV_OPW; ++o) {
          float t = acc[o][r];
          t += bf2f(w[o][i][0]) * a[0];
          t += bf2f(w[o][i][1]) * a[1];
          t += bf2f(w[o][i][2]) * a[2];
          t += bf2f(w[o][i][3]) * a[3];
          t += bf2f(w[o][i][4]) * c[0];
          t += bf2f(w[o][i][5]) * c[1];
          t += bf2f(w[o][i][6]) * c[2];
          t += bf2f(w[o][i][7]) * c[3];
          acc[o][r] = t;
        }
      }
    }
  }
#pragma unroll
  for (int o = 0; o < GV_OPW; ++o) {
    const int n = n0 + o;
    if (n >= N) break;
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
      if (r < R) {
        const float s = wave_sum(acc[o][r]);
        if (lane == 0) {
          const float v = s + b[n];
          y[(int64_t)r * N + n] = act_out ? silu(v) : v;
        }
      }
  }
}

constexpr int PT = 4;   // tokens per patch-embed workgroup (1280 tokens: 320 workgroups)
constexpr int MAXC = 64;

// Each thread owns 4 output columns and produces them for the workgroup's PT
// tokens, so a weight row group is read once per PT tokens; the weights come
// in 16-byte pieces of 8 channels (C a multiple of 8), one round of loads per
// 8 channels rather than per channel.
__global__ __launch_bounds__(256) void patch_embed_kernel(const float* __restrict__ lat, int C, int N,
                                                          const bf16_t* __restrict__ Wp,
                                                          const float* __restrict__ bp,
                                                          float* __restrict__ x, int D) {
  __shared__ float sl[MAXC * PT];
  const int b = blockIdx.y, t0 = wg_x() * PT;
  for (int i = threadIdx.x; i < C * PT; i += 256) {
    const int c = i / PT, tt = i % PT;
    sl[i] = t0 + tt < N ? lat[((int64_t)b * C + c) * N + t0 + tt] : 0.f;
  }
  __syncthreads();
  for (int d = threadIdx.x * 4; d < D; d += 1024) {
    float acc[PT][4];
    const float4 bias = *reinterpret_cast<const float4*>(bp + d);
#pragma unroll
    for (int tt = 0; tt < PT; ++tt) {
      acc[tt][0] = bias.x; acc[tt][1] = bias.y; acc[tt][2] = bias.z; acc[tt][3] = bias.w;
    }
    for (int c0 = 0; c0 < C; c0 += 8) {
      u16x8 w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const u16x8*>(Wp + (int64_t)(d + e) * C + c0);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int tt = 0; tt < PT; ++tt) {
          const float l = sl[(c0 + j) * PT + tt];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tt][e] += bf2f(w[e][j]) * l;
        }
    }
#pragma unroll
    for (int tt = 0; tt < PT; ++tt)
      if (t0 + tt < N)
        *reinterpret_cast<float4*>(x + ((int64_t)b * N + t0 + tt) * D + d) =
            make_float4(acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]);
  }
}

// Counter-based generator: Philox-4x32 with 10 rounds (Salmon, Moraes, Dror,
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011). A round
// multiplies words 0 and 2 by the two round constants (64-bit products), and
// the new words are (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)); the key advances by the two Weyl increments between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const u32x4 n = {(uint32_t)(p1 >> 32) ^ c[1] ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c[3] ^ k1,
                     (uint32_t)p0};
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Standard-normal noise of latent element i of batch lane b at step k:
// counter (i / 4, b, k, 0), key (seed low, high); element i takes the word
// pair (i mod 4) / 2 as two 24-bit uniforms in (0, 1] and the Box-Muller
// transform, cosine for even i, sine for odd i.
__device__ __forceinline__ float latent_noise(uint32_t i, uint32_t b, uint32_t k, uint32_t k0, uint32_t k1) {
  const u32x4 w = philox4x32_10(u32x4{i >> 2, b, k, 0u}, k0, k1);
  const int p = (i >> 1) & 1;
  const float ua = (float)((w[2 * p] >> 8) + 1u) * 0x1p-24f;
  const float ub = (float)((w[2 * p + 1] >> 8) + 1u) * 0x1p-24f;
  const float r = sqrtf(-2.f * logf(ua));
  const float th = 6.28318530717958647692f * ub;
  return r * ((i & 1) ? sinf(th) : cosf(th));
}

__global__ void philox_fill_kernel(uint32_t* __restrict__ out, int64_t n, uint32_t g0, uint32_t lane,
                                   uint32_t step, uint32_t k0, uint32_t k1) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n) return;
  const u32x4 w = philox4x32_10(u32x4{g0 + (uint32_t)g, lane, step, 0u}, k0, k1);
  *reinterpret_cast<u32x4*>(out + 4 * g) = w;
}

// Output head on the modulated, normalised rows h (bf16 [B*N, D]) fused with
// the sampler update: MFMA 16x16x32, one workgroup per 16 tokens, its 4 waves
// each taking a quarter of the D-long dot products (all of a wave's operand
// loads requested before its MFMAs), the quarters added in wave order through
// LDS; lane l holds token (l % 16) and channels 4 (l / 16) + {0..3} of a
// 16-channel group. Euler: x' = x + (s' - s) v. Re-noising: x' = (1 - s')
// (x - s v) + s' eps, eps from latent_noise (element index c * N + token
// within the lane).
constexpr int HE_KQ = 12;  // 32-deep k-steps a wave requests at once

__global__ __launch_bounds__(256) void head_euler_kernel(
    const bf16_t* __restrict__ h, int B, int N, int D, const bf16_t* __restrict__ Wh,
    const float* __restrict__ bh, int Co, const float* lat_cur, float* lat_next,
    const float* __restrict__ motion, int nmt, float sigma, float sigma_next, SamplerArgs sa) {
  __shared__ f32x4 part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = wg_x() * 16;
  const int lr = lane & 15, lq = lane >> 4;
  const int row = min(t0 + lr, B * N - 1);
  const int kq = D / 4;  // this wave's k range [wave kq, (wave + 1) kq)
  const bf16_t* hp = h + (int64_t)row * D + wave * kq + 8 * lq;
  const float dsig = sigma_next - sigma;
  for (int cg = 0; cg < Co; cg += 16) {
    const bf16_t* wp = Wh + (int64_t)(cg + lr) * D + wave * kq + 8 * lq;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < kq; k0 += 32 * HE_KQ) {
      bf16x8 a[HE_KQ], w[HE_KQ];
#pragma unroll
      for (int i = 0; i < HE_KQ; ++i)
        if (k0 + 32 * i < kq) {
          w[i] = *reinterpret_cast<const bf16x8*>(wp + k0 + 32 * i);
          a[i] = *reinterpret_cast<const bf16x8*>(hp + k0 + 32 * i);
        }
#pragma unroll
      for (int i = 0; i < HE_KQ; ++i)
        if (k0 + 32 * i < kq) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[i], a[i], acc, 0, 0, 0);
    }
    mfma_drain(acc);
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && t0 + lr < B * N) {
      f32x4 v4 = part[0][lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const f32x4 p = part[q][lane];
        v4[0] += p[0];
        v4[1] += p[1];
        v4[2] += p[2];
        v4[3] += p[3];
      }
      const int b = (t0 + lr) / N, tok = (t0 + lr) % N;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int co = cg + 4 * lq + i;
        const int64_t idx = ((int64_t)b * Co + co) * N + tok;
        if (tok < nmt) {
          lat_next[idx] = motion[((int64_t)b * Co + co) * nmt + tok];
        } else {
          const float v = v4[i] + bh[co];
          if (sa.renoise) {
            const float eps = latent_noise((uint32_t)(co * N + tok), (uint32_t)b, sa.step, sa.k0, sa.k1);
            lat_next[idx] = (1.f - sigma_next) * (lat_cur[idx] - sigma * v) + sigma_next * eps;
          } else {
            lat_next[idx] = lat_cur[idx] + dsig * v;
          }
        }
      }
    }
    __syncthreads();  // part[] is reused by the next channel group
  }
}

// Float32 form of the head update (debug precision): one thread per latent
// element (lane, channel, token), v = h[row] . W_h[co] + b_h[co] in float32.
__global__ __launch_bounds__(256) void head_euler_f32_kernel(
    const float* __restrict__ h, int B, int N, int D, const bf16_t* __restrict__ Wh,
    const float* __restrict__ bh, int Co, const float* lat_cur, float* lat_next,
    const float* __restrict__ motion, int nmt, float sigma, float sigma_next, SamplerArgs sa) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * Co * N) return;
  const int tok = (int)(i % N), co = (int)((i / N) % Co), b = (int)(i / ((int64_t)N * Co));
  if (tok < nmt) {
    lat_next[i] = motion[((int64_t)b * Co + co) * nmt + tok];
    return;
  }
  const float* hr = h + ((int64_t)b * N + tok) * D;
  const bf16_t* wr = Wh + (int64_t)co * D;
  float v = 0.f;
  for (int d = 0; d < D; ++d) v = fmaf(hr[d], bf2f(wr[d]), v);
  v += bh[co];
  if (sa.renoise) {
    const float eps = latent_noise((uint32_t)(co * N + tok), (uint32_t)b, sa.step, sa.k0, sa.k1);
    lat_next[i] = (1.f - sigma_next) * (lat_cur[i] - sigma * v) + sigma_next * eps;
  } else {
    lat_next[i] = lat_cur[i] + (sigma_next - sigma) * v;
  }
}

__global__ void pin_motion_kernel(const float* __restrict__ lat, const float* __restrict__ motion,
                                  float* __restrict__ out, int64_t total, int N, int nmt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bc = i / N;
  const int t = (int)(i % N);
  out[i] = t < nmt ? motion[bc * nmt + t] : lat[i];
}

__global__ void f32_to_bf16_kernel(const float* __restrict__ in, bf16_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = f2bf(in[i]);
}

// Clock probe: every wave issues `iters` groups of four independent bf16
// MFMAs (so the matrix core never waits on a result); wave 0 reads the shader
// cycle counter and the constant-rate wall clock before and after the
// workgroup's loops. out[4 wg + {0,1,2,3}] = cycles start, end, wall start,
// end. The accumulators are stored only when `sink` is set (never by the
// host), which keeps the MFMAs from being removed.
__global__ __launch_bounds__(256) void clock_probe_kernel(uint64_t* __restrict__ out, int iters, int sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  __syncthreads();
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  mfma_drain(acc[3]);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    out[4 * blockIdx.x] = t0;
    out[4 * blockIdx.x + 1] = t1;
    out[4 * blockIdx.x + 2] = r0;
    out[4 * blockIdx.x + 3] = r1;
  }
  if (sink) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) v += acc[k][r];
    reinterpret_cast<float*>(out)[threadIdx.x] = v;
  }
}

}  // namespace

hipError_t clock_probe(uint64_t* out, int n_wg, int iters, hipStream_t s) {
  if (!out || n_wg < 1 || iters < 1) return hipErrorInvalidValue;
  launch_timed(clock_probe_kernel, n_wg, 256, s, out, iters, 0);
  return hipGetLastError();
}

hipError_t head_euler_f32(const float* h, int B, int N, int D, const bf16_t* Wh, const float* bh, int Co,
                          const float* lat_cur, float* lat_next, const float* motion, int n_motion_tok,
                          float sigma, float sigma_next, const SamplerArgs& sa, hipStream_t s) {
  const int64_t total = (int64_t)B * Co * N;
  if (total <= 0) return hipSuccess;
  launch_timed(head_euler_f32_kernel, (unsigned)((total + 255) / 256), 256, s, h, B, N, D, Wh, bh, Co, lat_cur, lat_next,
               motion, n_motion_tok, sigma, sigma_next, sa);
  return hipGetLastError();
}

hipError_t rope_table(float* cos_t, float* sin_t, int F, int H, int W, int head_dim, double theta,
                      hipStream_t s) {
  const int half = head_dim / 2, nr = head_dim / 6, nf = half - 2 * nr;
  const int64_t total = (int64_t)F * H * W * half;
  launch_timed(rope_table_kernel, (unsigned)((total + 255) / 256), 256, s, cos_t, sin_t, F, H, W, half, nf, nr,
               theta);
  return hipGetLastError();
}

hipError_t sinusoid(float* out, const float* t_host, int R, int dim, hipStream_t s) {
  if (R <= 0 || R > MAXR || dim % 2) return hipErrorInvalidValue;
  Times ts{};
  for (int r = 0; r < R; ++r) ts.t[r] = t_host[r];
  launch_timed(sinusoid_kernel, (R * dim + 255) / 256, 256, s, out, ts, R, dim);
  return hipGetLastError();
}

hipError_t gemv_bf16(const float* x, int R, int K, const bf16_t* W, const float* b, float* y, int N,
                     int act_in, int act_out, hipStream_t s) {
  if (R <= 0 || R > MAXR || K % 8 || (size_t)R * K * 4 > 65536) return hipErrorInvalidValue;
  launch_timed_lds(gemv_kernel, (N + 15) / 16, 256, (size_t)R * K * 4, s, x, R, K, W, b, y, N, act_in, act_out);
  return hipGetLastError();
}

hipError_t patch_embed(const float* lat, int B, int C, int N, const bf16_t* Wp, const float* bp,
                       float* x, int D, hipStream_t s) {
  if (C > MAXC || C % 8 || D % 4 || ((uintptr_t)Wp & 15)) return hipErrorInvalidValue;
  dim3 grid((N + PT - 1) / PT, B);
  launch_timed(patch_embed_kernel, grid, 256, s, lat, C, N, Wp, bp, x, D);
  return hipGetLastError();
}

hipError_t head_euler(const bf16_t* h, int B, int N, int D, const bf16_t* Wh, const float* bh, int Co,
                      const float* lat_cur, float* lat_next, const float* motion, int n_motion_tok,
                      float sigma, float sigma_next, const SamplerArgs& sa, hipStream_t s) {
  if (D % 128 || Co % 16) return hipErrorInvalidValue;
  launch_timed(head_euler_kernel, (B * N + 15) / 16, 256, s, h, B, N, D, Wh, bh, Co, lat_cur, lat_next, motion,
               n_motion_tok, sigma, sigma_next, sa);
  return hipGetLastError();
}

hipError_t philox_fill(uint32_t* out, int64_t n_groups, uint32_t first_group, uint32_t lane, uint32_t step,
                       uint64_t seed, hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  launch_timed(philox_fill_kernel, (unsigned)((n_groups + 255) / 256), 256, s, out, n_groups, first_group, lane, step,
               (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError();
}

hipError_t pin_motion(const float* lat, const float* motion, float* out, int BC, int N,
                      int n_motion_tok, hipStream_t s) {
  const int64_t total = (int64_t)BC * N;
  launch_timed(pin_motion_kernel, (unsigned)((total + 255) / 256), 256, s, lat, motion, out, total, N,
               n_motion_tok);
  return hipGetLastError();
}

hipError_t f32_to_bf16(const float* in, bf16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  launch_timed(f32_to_bf16_kernel, (unsigned)((n + 255) / 256), 256, s, in, out, n);
  return hipGetLastError();
}

hipError_t set_wg_reverse_misc(int r) { return set_wg_reverse(r); }

}  // namespace fh
