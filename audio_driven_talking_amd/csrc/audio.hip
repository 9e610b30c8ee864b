// Audio projection front end: speech-encoder states -> the DiT's audio tokens.
//
// The gizai:flashhead page (overview) makes 5 latent frames of 32 audio tokens
// from 5 states around each of a slice's 33 frames, taken from wav2vec 2.0's
// 12 layers at 200 frames; its type listing names the layers proj1, proj1vf,
// proj2, proj3 and projNorm. The arrangement below is the plain reading of
// that: a frame's feature is its 5-state window (clamped at the ends of the
// states) flattened in (offset, layer, channel) order; latent frame 0 is video
// frame 0, latent frame i >= 1 the mean of video frames s(i-1)+1 .. s i (s the
// VAE's temporal stride); proj1 (latent frame 0) and proj1vf (the others),
// SiLU, proj2, SiLU, proj3 to tokens x D, LayerNorm with gain and bias.
//
// Kernels: the window gather with the group mean (bf16 GEMM operand, rows
// latent-frame-major so proj1 and proj1vf each read one contiguous block),
// split-K GEMMs on the bf16 MFMA kernel for the long reductions (K = 5 L C is
// 46080 for the Lite sizes, with M the number of latent frames), a reduction
// of the split parts with bias and activation, and the float32 LayerNorm.
#include <hip/hip_runtime.h>

#include "fh_kernels.h"

namespace fh {
namespace {

// X[(i * B + b)][(d * L + l) * C + c] = mean over video frames f of latent frame i of
// states[b][l][clamp(T - V + f + d - W/2)][c], rounded to bf16
__global__ __launch_bounds__(256) void audio_features_kernel(const float* __restrict__ states, int B, int L, int T,
                                                             int C, int W, int V, int stride, int LF,
                                                             bf16_t* __restrict__ X) {
  const int64_t F = (int64_t)W * L * C;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)LF * B * F) return;
  const int64_t k = i % F;
  const int row = (int)(i / F), lf = row / B, b = row % B;
  const int c = (int)(k % C), l = (int)((k / C) % L), d = (int)(k / ((int64_t)C * L));
  const int f0 = lf == 0 ? 0 : stride * (lf - 1) + 1, nf = lf == 0 ? 1 : stride;
  const float* sl = states + ((int64_t)b * L + l) * T * C + c;
  float sum = 0.f;
  for (int f = f0; f < f0 + nf; ++f) {
    const int t = min(max(T - V + f + d - W / 2, 0), T - 1);
    sum += sl[(int64_t)t * C];
  }
  X[i] = f2bf(sum / (float)nf);
}

// out[row(m)][n] = act(sum_s part[s][m][n] + bias[n]), parts added in index order;
// row(m) = (m % group) * ngroups + m / group (the identity for group = M);
// act: 0 none, 1 SiLU; out is float32 (out_f) or bf16 (out_b)
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                        const float* __restrict__ bias, int act, int group,
                                                        int ngroups, float* __restrict__ out_f,
                                                        bf16_t* __restrict__ out_b) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float v = part[i];
  for (int s = 1; s < splits; ++s) v += part[s * MN + i];
  v += bias[n];
  if (act == 1) v = v / (1.0f + expf(-v));
  const int64_t o = ((int64_t)(m % group) * ngroups + m / group) * N + n;
  if (out_f) out_f[o] = v;
  else out_b[o] = f2bf(v);
}

// The same for many parts: one wave per output element, lane l adding parts
// l, l + 64, ... in index order, then the 64 lane sums by a fixed butterfly
// (lane 0's sum is stored), so the loads of all parts are in flight at once
// instead of one after the other.
__global__ __launch_bounds__(256) void sum_parts_wide_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                             const float* __restrict__ bias, int act, int group,
                                                             int ngroups, float* __restrict__ out_f,
                                                             bf16_t* __restrict__ out_b) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t MN = (int64_t)M * N;
  if (i >= MN) return;  // whole waves
  const int lane = threadIdx.x & 63;
  float v = 0.f;
  for (int s = lane; s < splits; s += 64) v += part[s * MN + i];
  v = wave_sum(v);
  if (lane) return;
  const int m = (int)(i / N), n = (int)(i % N);
  v += bias[n];
  if (act == 1) v = v / (1.0f + expf(-v));
  const int64_t o = ((int64_t)(m % group) * ngroups + m / group) * N + n;
  if (out_f) out_f[o] = v;
  else out_b[o] = f2bf(v);
}

}  // namespace

hipError_t audio_features(const float* states, int B, int L, int T, int C, int W, int V, int stride, int LF,
                          bf16_t* X, hipStream_t s) {
  const int64_t total = (int64_t)LF * B * W * L * C;
  if (total <= 0) return hipSuccess;
  if (T <= 0 || stride <= 0 || (V - 1) != stride * (LF - 1)) return hipErrorInvalidValue;
  launch_timed(audio_features_kernel, (unsigned)((total + 255) / 256), 256, s, states, B, L, T, C, W, V, stride, LF, X);
  return hipGetLastError();
}

hipError_t sum_parts(const float* part, int splits, int M, int N, const float* bias, int act, int group,
                     int ngroups, float* out_f, bf16_t* out_b, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  if (total <= 0) return hipSuccess;
  if (splits < 1 || !bias || (!out_f && !out_b) || group <= 0 || ngroups <= 0 || (int64_t)group * ngroups != M)
    return hipErrorInvalidValue;
  if (splits >= 16 && total <= ((int64_t)1 << 24))
    launch_timed(sum_parts_wide_kernel, (unsigned)((total * 64 + 255) / 256), 256, s, part, splits, M, N, bias, act, group,
                 ngroups, out_f, out_b);
  else
    launch_timed(sum_parts_kernel, (unsigned)((total + 255) / 256), 256, s, part, splits, M, N, bias, act, group, ngroups,
                 out_f, out_b);
  return hipGetLastError();
}

}  // namespace fh
