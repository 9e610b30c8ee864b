// bf16 GEMM on gfx950 MFMA: C[M,N] = A[M,K] * W[N,K]^T with fp32 accumulation
// and fused epilogues (bias, tanh-GELU, gated / plain fp32 residual, split
// row-major / transposed store).
//
// Both operands are K-contiguous (activations [tokens, K], weights [out, in]).
// The MFMA is issued as W-fragment x A-fragment so that each lane of a 32x32
// result holds 4 consecutive output columns of one row: the epilogue then
// reads/writes 16-byte fp32 vectors (or 8-byte bf16 vectors).
//
// Workgroup tile BM x BN, K-slabs of 64, 256 threads = 4 waves in 2x2, each
// wave (BM/2) x (BN/2) of MFMA 32x32x16 blocks.
// Operand slabs go global -> LDS directly (global_load_lds_dwordx4: each wave
// instruction fills 1 KB = 8 rows x 128 B), NS slabs deep, so NS-1 slabs are
// in flight while one is multiplied; one barrier per slab. Inside a 128-byte
// row the 16-byte chunks are XOR-swizzled by (row & 7), which makes the
// fragment reads of 8 consecutive rows hit 8 different bank groups.
// Tile order is XCD-aware: the grid is padded to a multiple of the 8 XCDs and
// each XCD gets a contiguous run of tiles, M fastest, so the tiles sharing a
// weight slab share an L2.
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int KALIGN = 64;  // K must be a multiple of this (either slab depth divides it)

template <int EPI>
__device__ __forceinline__ void epilogue4(const EpiArgs& ep, int m, int n, f32x4 v) {
  const float4 b = *reinterpret_cast<const float4*>(ep.bias + n);
  float c0 = v[0] + b.x, c1 = v[1] + b.y, c2 = v[2] + b.z, c3 = v[3] + b.w;
  if constexpr (EPI == EPI_BF16 || EPI == EPI_GELU_BF16) {
    if constexpr (EPI == EPI_GELU_BF16) {
      c0 = gelu_tanh(c0); c1 = gelu_tanh(c1); c2 = gelu_tanh(c2); c3 = gelu_tanh(c3);
    }
    const u32x2 w = {pack2bf(c0, c1), pack2bf(c2, c3)};
    *reinterpret_cast<u32x2*>(ep.out_bf + (int64_t)m * ep.ldo + n) = w;
  } else if constexpr (EPI == EPI_GATED_RES || EPI == EPI_RES) {
    f32x4* xp = reinterpret_cast<f32x4*>(ep.x + (int64_t)m * ep.ldx + n);
    f32x4 x = *xp;
    if constexpr (EPI == EPI_GATED_RES) {
      const int lane = m / ep.rows_per_lane;
      const float4 gt = *reinterpret_cast<const float4*>(ep.gate_tab + n);
      const float4 ge = *reinterpret_cast<const float4*>(ep.gate_e0 + (int64_t)lane * ep.gate_stride + n);
      c0 *= gt.x + ge.x; c1 *= gt.y + ge.y; c2 *= gt.z + ge.z; c3 *= gt.w + ge.w;
    }
    x[0] += c0; x[1] += c1; x[2] += c2; x[3] += c3;
    *xp = x;
  } else {  // EPI_SPLIT_T
    if (n < ep.split) {
      const u32x2 w = {pack2bf(c0, c1), pack2bf(c2, c3)};
      *reinterpret_cast<u32x2*>(ep.out_bf + (int64_t)m * ep.ldo + n) = w;
    } else {
      const int lane = m / ep.rows_per_lane, t = m - lane * ep.rows_per_lane;
      bf16_t* o = ep.out_t + ((int64_t)lane * ep.t_cols + (n - ep.split)) * ep.rows_per_lane + t;
      o[0] = f2bf(c0);
      o[ep.rows_per_lane] = f2bf(c1);
      o[2 * ep.rows_per_lane] = f2bf(c2);
      o[3 * ep.rows_per_lane] = f2bf(c3);
    }
  }
}

template <int BM, int BN, int BK, int NS>
constexpr int smem_bytes() { return NS * (BM + BN) * BK * 2; }

// XOR swizzle of the 16-byte chunk index inside an LDS row. gfx950 serves a
// 16-byte LDS read in groups of 16 lanes across 64 banks (a 256-byte window),
// so the 16 consecutive rows a fragment read touches at one logical chunk
// must land on 16 different 16-byte slots of that window: rows of 128 B
// (K-slab 64) already alternate between the two halves by parity and XOR
// with (row >> 1) & 7; rows of 64 B (K-slab 32) take the quarter from
// row & 3 and XOR with (row >> 2) & 3.
template <int BK>
__device__ __forceinline__ int swz(int row) { return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3); }

template <int EPI, int BM, int BN, int BK, int NS>
__global__ __launch_bounds__(256, (smem_bytes<BM, BN, BK, NS>() <= 80 * 1024) ? 2 : 1)
void gemm_bf16_nt(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw,
                  int M, int N, int K, int tiles_m, int tiles, EpiArgs ep) {
  constexpr int ROWB = BK * 2;         // bytes per LDS row of a slab
  constexpr int CH = BK / 8;           // 16-byte chunks per row
  constexpr int RG = 64 / CH;          // rows per 1 KB DMA group
  constexpr int MI = BM / 64;          // 32-row activation blocks per wave
  constexpr int NI = BN / 64;          // 32-row weight blocks per wave
  constexpr int GA = BM / RG / 4;      // 1 KB DMA groups per wave per slab, activations
  constexpr int GW = BN / RG / 4;      // ... weights
  constexpr int SLAB = (BM + BN) * ROWB;
  constexpr int INFLIGHT = (NS - 2) * (GA + GW);  // DMAs of younger slabs allowed in flight
  static_assert(GA >= 1 && GW >= 1 && INFLIGHT < 64, "tile shape");
  __shared__ __attribute__((aligned(1024))) char smem[NS * SLAB];

  int bid = blockIdx.x;
  const int per_xcd = gridDim.x >> 3;
  bid = (bid & 7) * per_xcd + (bid >> 3);
  if (bid >= tiles) return;
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  // DMA: lane fills LDS row r = RG g + lane/CH, physical chunk lane%CH, which
  // holds logical chunk (lane%CH) ^ swz(r)
  const int drow = lane / CH;
  const bf16_t* ga[GA];
  const bf16_t* gw[GW];
#pragma unroll
  for (int i = 0; i < GA; ++i) {
    const int r = RG * (wave + 4 * i) + drow;
    ga[i] = A + (int64_t)min(m0 + r, M - 1) * lda + ((lane % CH) ^ swz<BK>(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int r = RG * (wave + 4 * i) + drow;
    gw[i] = W + (int64_t)(n0 + r) * ldw + ((lane % CH) ^ swz<BK>(r)) * 8;
  }

  auto issue = [&](int buf, int k0) {
    char* sa = smem + buf * SLAB;
    char* sw = sa + BM * ROWB;
#pragma unroll
    for (int i = 0; i < GA; ++i) dma16(ga[i] + k0, sa + (wave + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < GW; ++i) dma16(gw[i] + k0, sw + (wave + 4 * i) * 1024);
  };

  f32x16 acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment rows: activations wm*BM/2 + 32 j + lr, weights wn*BN/2 + 32 i + lr
  const int xr = swz<BK>(lr);
  auto compute = [&](int buf) {
    const char* sa = smem + buf * SLAB + (wm * (BM / 2) + lr) * ROWB;
    const char* sw = smem + buf * SLAB + BM * ROWB + (wn * (BN / 2) + lr) * ROWB;
    // fragments of k-step kk+1 are read while the MFMAs of k-step kk run
    bf16x8 wf[2][NI], af[2][MI];
    auto read = [&](int set, int kk) {
      const int off = ((2 * kk + lh) ^ xr) * 16;
#pragma unroll
      for (int i = 0; i < NI; ++i) wf[set][i] = *reinterpret_cast<const bf16x8*>(sw + i * 32 * ROWB + off);
#pragma unroll
      for (int j = 0; j < MI; ++j) af[set][j] = *reinterpret_cast<const bf16x8*>(sa + j * 32 * ROWB + off);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read((kk + 1) & 1, kk + 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the next reads ahead of these MFMAs
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk & 1][i], af[kk & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int KT = K / BK;
  // prologue: slabs 0 .. NS-2 in flight (slabs past the end re-fetch the last
  // one into buffers nobody reads, keeping the wait count uniform)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, KT - 1) * BK);
  for (int kt = 0; kt < KT; ++kt) {
    wait_vm<INFLIGHT>();   // this wave's DMAs of slab kt have landed
    barrier();             // everyone's have; everyone is done with slab kt-1
    issue((kt + NS - 1) % NS, min(kt + NS - 1, KT - 1) * BK);
    compute(kt % NS);
  }
  wait_vm<0>();

  // result (i, j): lane holds row m = m0 + wm*BM/2 + j*32 + lr and columns
  // n = n0 + wn*BN/2 + i*32 + 8g + 4lh + {0..3} in acc[i][j][4g .. 4g+3]
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int m = m0 + wm * (BM / 2) + j * 32 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / 2) + i * 32 + 8 * g + 4 * lh;
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        epilogue4<EPI>(ep, m, n, v);
      }
  }
}

template <int BM, int BN, int BK, int NS>
hipError_t launch(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                  const EpiArgs& ep, hipStream_t s) {
  if (N % BN) return hipErrorInvalidValue;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = tiles_m * (N / BN);
  const dim3 grid((tiles + 7) / 8 * 8), block(256);
  switch (epi) {
    case EPI_BF16: gemm_bf16_nt<EPI_BF16, BM, BN, BK, NS><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, tiles, ep); break;
    case EPI_GELU_BF16: gemm_bf16_nt<EPI_GELU_BF16, BM, BN, BK, NS><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, tiles, ep); break;
    case EPI_GATED_RES: gemm_bf16_nt<EPI_GATED_RES, BM, BN, BK, NS><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, tiles, ep); break;
    case EPI_RES: gemm_bf16_nt<EPI_RES, BM, BN, BK, NS><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, tiles, ep); break;
    case EPI_SPLIT_T: gemm_bf16_nt<EPI_SPLIT_T, BM, BN, BK, NS><<<grid, block, 0, s>>>(A, lda, W, ldw, M, N, K, tiles_m, tiles, ep); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Tile choice from measurements of the slice shapes on MI355X with weights
// cold in HBM (as in a 30-block slice): big tiles (less L2->LDS traffic per
// FLOP) where they still give enough workgroups, smaller ones otherwise.
int gemm_tile_choice(int M, int N, int K) {
  const int64_t t256 = (int64_t)((M + 255) / 256) * (N / 256);
  if (N % 256 == 0 && N >= 4096 && t256 >= 170) return 0;  // 256x256, K-slab 64, 2 stages
  if (N <= 2048 && M <= 1536) return K >= 4096 ? 2 : 3;     // 128x64 k64 s4 | 64x64 k64 s4
  return 1;                                                 // 128x128 k32 s4
}

hipError_t gemm_bf16(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                     const EpiArgs& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % 128 || K % KALIGN || lda % 8 || ldw % 8) return hipErrorInvalidValue;
  switch (gemm_tile_choice(M, N, K)) {
    case 0: return launch<256, 256, 64, 2>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case 1: return launch<128, 128, 32, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case 2: return launch<128, 64, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
    default: return launch<64, 64, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
  }
}

}  // namespace fh
