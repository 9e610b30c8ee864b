// Attention on gfx950 MFMA 32x32x16 bf16, head_dim 128, fp32 online softmax.
//
// Formulation: each wave owns 32 queries and computes S^T = K Q^T (keys on
// the MFMA rows, queries on the columns), so a lane holds 16 scores of ONE
// query. The running max/sum of the online softmax are then per-lane scalars
// (one exchange with lane^32 for the block max), and O^T = V^T P^T reuses the
// score registers directly as the B fragment: the key order inside a
// 16-wide k-step is permuted the same way on the V^T side, which the MFMA
// sum does not see. Values arrive transposed ([dim, keys]) from the
// projection epilogue, so V^T tiles are plain row copies.
//
// flash_attn: 128 queries (4 waves) per workgroup; K and V^T blocks of 64
// keys are staged in padded LDS, double-buffered, the next block fetched to
// registers during the current one.
// cross_attn: short key ranges (32 audio tokens per latent frame, or all of
// them), fragments loaded straight from global memory, no LDS.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int HD = 128;
constexpr int QT = 128;
constexpr int KB = 64;
constexpr int KR = HD + 8;  // padded K row in LDS (bf16): 272 bytes
constexpr int VR = KB + 4;  // padded V^T row in LDS (bf16): 136 bytes

__device__ __forceinline__ bf16x8 load_v_frag(const bf16_t* p) {
  // keys {0..3} and {8..11} relative to p (see the key permutation above)
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  const u32x4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 p_frag(const f32x16& st, int u) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)st[8 * u + e];
  return f;
}

__device__ __forceinline__ void store_o(bf16_t* orow, const f32x16 (&acc)[4], float inv, int lh) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 w;
      w.x = pack2bf(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv);
      w.y = pack2bf(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * g + 4 * lh) = w;
    }
}

__global__ __launch_bounds__(256, 1) void flash_attn_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ k, int ldk,
    const bf16_t* __restrict__ vt, bf16_t* __restrict__ o, int ldo, int N, int D,
    float scale_log2) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KB * KR];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][HD * VR];
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = blockIdx.x * QT + wave * 32;

  bf16x8 qf[8];
  {
    const int qrow = min(q0 + lr, N - 1);
    const bf16_t* qp = q + ((int64_t)b * N + qrow) * ldq + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  // staging: K block 64 rows x 16 chunks, V^T block 128 rows x 8 chunks
  const int kc = tid & 15, kr = tid >> 4;
  const int vc = tid & 7, vr = tid >> 3;
  const bf16_t* kbase = k + (int64_t)b * N * ldk + h * HD + kc * 8;
  const bf16_t* vbase = vt + ((int64_t)b * D + h * HD) * N + vc * 8;
  u32x4 gk[4], gv[4];
  auto gload = [&](int kb0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kb0 + kr + 16 * i, N - 1);
      gk[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * ldk);
    }
    const bool in = kb0 + vc * 8 < N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      gv[i] = in ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)(vr + 32 * i) * N + kb0)
                 : u32x4{0u, 0u, 0u, 0u};
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sK[buf][(kr + 16 * i) * KR + kc * 8]) = gk[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16_t* p = &sV[buf][(vr + 32 * i) * VR + vc * 8];
      reinterpret_cast<u32x2*>(p)[0] = u32x2{gv[i].x, gv[i].y};
      reinterpret_cast<u32x2*>(p)[1] = u32x2{gv[i].z, gv[i].w};
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nkb = (N + KB - 1) / KB;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload((kb + 1) * KB);

    f32x16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
      const bf16_t* kp = &sK[cur][(32 * t + lr) * KR + 8 * lh];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + 16 * s),
                                                        qf[s], st[t], 0, 0, 0);
    }
    float mx = -INFINITY;
    const bool tail = (kb + 1) * KB > N;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = st[t][r] * scale_log2;
        if (tail) {
          const int key = kb * KB + 32 * t + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (key >= N) v = -INFINITY;
        }
        st[t][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(st[t][r] - m_new);
        st[t][r] = p;
        ps += p;
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pf = p_frag(st[t], u);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 vf = load_v_frag(&sV[cur][(32 * dt + lr) * VR + 32 * t + 16 * u + 4 * lh]);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[dt], 0, 0, 0);
        }
      }
    if (kb + 1 < nkb) sstore(cur ^ 1);
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 32, 64);
  if (q0 + lr < N) store_o(o + ((int64_t)b * N + q0 + lr) * ldo + h * HD, acc, 1.f / l_run, lh);
}

__global__ __launch_bounds__(256) void cross_attn_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ kc, int ldk,
    const bf16_t* __restrict__ vct, bf16_t* __restrict__ o, int ldo, int N, int La, int D, int hw,
    int apf, int full, float scale_log2) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = blockIdx.x * QT + wave * 32;
  if (q0 >= N) return;

  bf16x8 qf[8];
  {
    const int qrow = min(q0 + lr, N - 1);
    const bf16_t* qp = q + ((int64_t)b * N + qrow) * ldq + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }
  const int k_lo = full ? 0 : (q0 / hw) * apf;
  const int k_hi = full ? La : k_lo + apf;

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = k_lo; k0 < k_hi; k0 += 32) {
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
    const bf16_t* kp = kc + ((int64_t)b * La + k0 + lr) * ldk + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + 16 * s),
                                                   qf[s], st, 0, 0, 0);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st[r] *= scale_log2;
      mx = fmaxf(mx, st[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f(st[r] - m_new);
      st[r] = p;
      ps += p;
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pf = p_frag(st, u);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16_t* vp = vct + ((int64_t)b * D + h * HD + 32 * dt + lr) * La + k0 + 16 * u + 4 * lh;
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_v_frag(vp), pf, acc[dt], 0, 0, 0);
      }
    }
  }
  l_run += __shfl_xor(l_run, 32, 64);
  if (q0 + lr < N) store_o(o + ((int64_t)b * N + q0 + lr) * ldo + h * HD, acc, 1.f / l_run, lh);
}

}  // namespace

hipError_t flash_attn(const bf16_t* q, int ldq, const bf16_t* k, int ldk, const bf16_t* vt,
                      bf16_t* o, int ldo, int B, int N, int n_heads, float scale, hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if (N % 8 || ldq % 8 || ldk % 8 || ldo % 4) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((N + QT - 1) / QT, n_heads, B);
  flash_attn_kernel<<<grid, 256, 0, s>>>(q, ldq, k, ldk, vt, o, ldo, N, n_heads * HD, scale_log2);
  return hipGetLastError();
}

hipError_t cross_attn(const bf16_t* q, int ldq, const bf16_t* kc, int ldk, const bf16_t* vct,
                      bf16_t* o, int ldo, int B, int N, int La, int hw, int apf, int full,
                      int n_heads, float scale, hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if (N % 32 || hw % 32 || apf % 32 || La % 32 || ldq % 8 || ldk % 8 || ldo % 4)
    return hipErrorInvalidValue;
  if (!full && (N / hw) * apf > La) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((N + QT - 1) / QT, n_heads, B);
  cross_attn_kernel<<<grid, 256, 0, s>>>(q, ldq, kc, ldk, vct, o, ldo, N, La, n_heads * HD, hw, apf,
                                         full, scale_log2);
  return hipGetLastError();
}

}  // namespace fh
