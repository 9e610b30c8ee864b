// bf16 GEMM on gfx950 MFMA: C[M,N] = A[M,K] * W[N,K]^T with fp32 accumulation
// and fused epilogues (bias, tanh-GELU, gated / plain fp32 residual, split
// row-major / transposed store).
//
// Both operands are K-contiguous (activations [tokens, K], weights [out, in]).
// The MFMA is issued as W-fragment x A-fragment so that each lane of the
// 32x32 result holds 4 consecutive output columns of one row: the epilogue
// then reads/writes 16-byte fp32 vectors (or 8-byte bf16 vectors).
//
// Tile: 128 (M) x 128 (N) x 64 (K), 256 threads = 4 waves in 2x2, each wave
// 64x64 = 2x2 MFMA 32x32x16 tiles. LDS is double-buffered, rows padded to
// 144 bytes so the fragment reads of 32 consecutive rows spread over all banks;
// the next K-slab is fetched into registers while the current one is used.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDR = BK + 8;  // padded LDS row, in bf16 elements

template <int EPI>
__device__ __forceinline__ void epilogue4(const EpiArgs ep, int m, int n, f32x4 v) {
  float4 b = *reinterpret_cast<const float4*>(ep.bias + n);
  float c0 = v[0] + b.x, c1 = v[1] + b.y, c2 = v[2] + b.z, c3 = v[3] + b.w;
  if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU_BF16) {
    if constexpr (EPI == EPI_GELU_BF16) {
      c0 = gelu_tanh(c0); c1 = gelu_tanh(c1); c2 = gelu_tanh(c2); c3 = gelu_tanh(c3);
    }
    uint2 w;
    w.x = pack2bf(c0, c1);
    w.y = pack2bf(c2, c3);
    *reinterpret_cast<uint2*>(ep.out_bf + (int64_t)m * ep.ldo + n) = w;
  } else if constexpr (EPI == EPI_GATED_RES || EPI == EPI_RES) {
    float4* xp = reinterpret_cast<float4*>(ep.x + (int64_t)m * ep.ldx + n);
    float4 x = *xp;
    if constexpr (EPI == EPI_GATED_RES) {
      int lane = m / ep.rows_per_lane;
      float4 gt = *reinterpret_cast<const float4*>(ep.gate_tab + n);
      float4 ge = *reinterpret_cast<const float4*>(ep.gate_e0 + (int64_t)lane * ep.gate_stride + n);
      c0 *= gt.x + ge.x; c1 *= gt.y + ge.y; c2 *= gt.z + ge.z; c3 *= gt.w + ge.w;
    }
    x.x += c0; x.y += c1; x.z += c2; x.w += c3;
    *xp = x;
  } else {  // EPI_SPLIT_T
    if (n < ep.split) {
      uint2 w;
      w.x = pack2bf(c0, c1);
      w.y = pack2bf(c2, c3);
      *reinterpret_cast<uint2*>(ep.out_bf + (int64_t)m * ep.ldo + n) = w;
    } else {
      int lane = m / ep.rows_per_lane, t = m - lane * ep.rows_per_lane;
      bf16_t* o = ep.out_t + ((int64_t)lane * ep.t_cols + (n - ep.split)) * ep.rows_per_lane + t;
      o[0] = f2bf(c0);
      o[ep.rows_per_lane] = f2bf(c1);
      o[2 * ep.rows_per_lane] = f2bf(c2);
      o[3 * ep.rows_per_lane] = f2bf(c3);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_nt(const bf16_t* __restrict__ A, int lda,
                                                        const bf16_t* __restrict__ W, int ldw, int M,
                                                        int N, int K, int tiles_m, EpiArgs ep) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][BN * LDR];

  // Tile order: workgroups are dealt round-robin to the 8 XCDs; give each XCD
  // a contiguous run of tiles, M fastest, so tiles sharing a weight slab sit
  // in the same L2.
  int bid = blockIdx.x;
  const int nt = gridDim.x;
  if ((nt & 7) == 0) bid = (bid & 7) * (nt >> 3) + (bid >> 3);
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  // global -> register staging: thread covers chunk c (8 bf16) of rows r0 + 32 i
  const int c = tid & 7, r0 = tid >> 3;
  const bf16_t* pa[4];
  const bf16_t* pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int ra = min(m0 + r0 + 32 * i, M - 1);
    pa[i] = A + (int64_t)ra * lda + c * 8;
    pw[i] = W + (int64_t)(n0 + r0 + 32 * i) * ldw + c * 8;
  }
  u32x4 ga[4], gw[4];
#define GEMM_GLOAD1(i, k0)                                      \
  ga[i] = *reinterpret_cast<const u32x4*>(pa[i] + (k0));        \
  gw[i] = *reinterpret_cast<const u32x4*>(pw[i] + (k0));
#define GEMM_GLOAD(k0) \
  GEMM_GLOAD1(0, k0) GEMM_GLOAD1(1, k0) GEMM_GLOAD1(2, k0) GEMM_GLOAD1(3, k0)
#define GEMM_SSTORE1(i, buf)                                                    \
  *reinterpret_cast<u32x4*>(&sA[buf][(r0 + 32 * i) * LDR + c * 8]) = ga[i];     \
  *reinterpret_cast<u32x4*>(&sW[buf][(r0 + 32 * i) * LDR + c * 8]) = gw[i];
#define GEMM_SSTORE(buf) \
  GEMM_SSTORE1(0, buf) GEMM_SSTORE1(1, buf) GEMM_SSTORE1(2, buf) GEMM_SSTORE1(3, buf)

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) { GEMM_GLOAD((kt + 1) * BK); }
    const bf16_t* a_base = &sA[cur][(wm * 64 + lr) * LDR + lh * 8];
    const bf16_t* w_base = &sW[cur][(wn * 64 + lr) * LDR + lh * 8];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 wf[2], af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        wf[i] = *reinterpret_cast<const bf16x8*>(w_base + i * 32 * LDR + kk * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        af[j] = *reinterpret_cast<const bf16x8*>(a_base + j * 32 * LDR + kk * 16);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) { GEMM_SSTORE(cur ^ 1); }
    __syncthreads();
  }

  // result (i, j): lane holds row m = m0 + wm*64 + j*32 + lr and columns
  // n = n0 + wn*64 + i*32 + 8g + 4lh + {0..3} in acc[i][j][4g .. 4g+3]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + j * 32 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + i * 32 + 8 * g + 4 * lh;
        f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        epilogue4<EPI>(ep, m, n, v);
      }
  }
}

}  // namespace

hipError_t gemm_bf16(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                     const EpiArgs& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % BN || K % BK || lda % 8 || ldw % 8) return hipErrorInvalidValue;
  const int tiles_m = (M + BM - 1) / BM;
  dim3 grid(tiles_m * (N / BN)), block(256);
  switch (epi) {
    case EPI_BF16: gemm_bf16_nt<EPI_BF16><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, ep); break;
    case EPI_GELU_BF16: gemm_bf16_nt<EPI_GELU_BF16><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, ep); break;
    case EPI_GATED_RES: gemm_bf16_nt<EPI_GATED_RES><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, ep); break;
    case EPI_RES: gemm_bf16_nt<EPI_RES><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, ep); break;
    case EPI_SPLIT_T: gemm_bf16_nt<EPI_SPLIT_T><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, ep); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fh
