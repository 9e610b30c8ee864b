// Video decoder after the denoiser on gfx950: the slice latent to 33 RGB
// frames through causal 3 x 3 x 3 convolutions (an assumed LTX-style layout:
// conv_in, three stages of a residual block and a depth-to-space up-sampling
// convolution, norm + SiLU, conv_out unfolded into 4 x 4 pixels).
//
// Numerics follow the audio-cpp page "SoulX-FlashHead", section "Variant
// boundaries": convolutions take F16 operands with F32 accumulation and
// store F16, the channel bias added in F32 to the F16-rounded sum before the
// final F16 cast; residual sums are stored in F16; the channel RMS norm
// accumulates in F32 and stores F16; the public latent and frames are F32.
//
// Activations are channels-last F16, [T][H][W][C]. A convolution is an
// implicit GEMM on the F16 MFMA (32x32x16): rows are output positions
// (M = T H W), columns output channels, and K = 27 C_in runs tap-major
// (tap = 9 dt + 3 dh + dw, then the input channel), which is exactly the
// kernel's [C_out][3][3][3][C_in] layout, so the weights are the B operand as
// stored. Each K-slab of 32 is DMA'd to LDS: every lane computes the source
// of its own 16-byte chunk (its output position shifted by the chunk's tap:
// frames before 0 clamp to frame 0, the causal padding; positions outside
// the frame read a zero row), so the shifted input is never materialised.
// The epilogue rounds and stores in the layer's own form: plain, plus a
// residual, depth to space into the next resolution, or the final pixels.
#include <algorithm>

#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int CBM = 128;   // output positions per tile
constexpr int CBK = 32;    // K per slab (64-byte LDS rows)
constexpr int CNS = 4;     // slab stages

// 16-byte chunk swizzle of 64-byte rows: the 16 rows a fragment read touches
// at one logical chunk take 16 distinct 16-byte slots of a 256-byte bank
// window (the quarter from row & 3, the XOR from (row >> 2) & 3)
__device__ __forceinline__ int cswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ float round16(float x) { return (float)(f16_t)x; }

// The layer's output of 4 consecutive channels n..n+3 of position m from their
// F32 sums: F16 sum, bias added in F32, F16, then stored in the layer's form.
template <int EPI>
__device__ __forceinline__ void store4(const ConvArgs& a, int m, int n, const float (&acc)[4]) {
  const int HW = a.H * a.W;
  const int t = m / HW, h = (m - t * HW) / a.W, w = m - t * HW - h * a.W;
  const f32x4 b = *reinterpret_cast<const f32x4*>(a.bias + n);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = round16(round16(acc[e]) + b[e]);
  if constexpr (EPI == CONV_PLAIN || EPI == CONV_RES) {
    f16_t* o = a.out + (int64_t)m * a.cout + n;
    if constexpr (EPI == CONV_RES) {
      const f16x4 r = *reinterpret_cast<const f16x4*>(a.res + (int64_t)m * a.cout + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] + (float)r[e];
    }
    const f16x4 y = {(f16_t)v[0], (f16_t)v[1], (f16_t)v[2], (f16_t)v[3]};
    *reinterpret_cast<f16x4*>(o) = y;
  } else if constexpr (EPI == CONV_UP) {
    // channel n = s C' + c (C' a multiple of 4: the 4 channels share s)
    const int cp = a.cout >> 3, s = n / cp, c = n - s * cp;
    const int t2 = 2 * t + (s >> 2) - 1, h2 = 2 * h + ((s >> 1) & 1), w2 = 2 * w + (s & 1);
    if (t2 >= 0) {
      f16_t* o = a.out + ((int64_t)(t2 * 2 * a.H + h2) * 2 * a.W + w2) * cp + c;
      const f16x4 y = {(f16_t)v[0], (f16_t)v[1], (f16_t)v[2], (f16_t)v[3]};
      *reinterpret_cast<f16x4*>(o) = y;
    }
  } else {
    // CONV_FRAMES: channel n = c 16 + 4 py + px -> pixel (4 h + py, 4 w + px) of colour c,
    // value (v + 1) / 2 clamped to [0, 1]
    const int c = n >> 4, py = (n >> 2) & 3;
    float* o = a.frames + ((int64_t)(c * a.T + t) * 4 * a.H + 4 * h + py) * 4 * a.W + 4 * w;
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf((v[e] + 1.f) * 0.5f, 0.f), 1.f);
    *reinterpret_cast<f32x4*>(o) = y;
  }
}

// EPI == CONV_PART: split K; workgroup split ks multiplies slabs [ks KT / splits,
// (ks + 1) KT / splits) and writes its raw F32 sums to part[ks][m][n]
template <int BN, int EPI>
__global__ __launch_bounds__(256) void conv3d_kernel(ConvArgs a, int tiles_m, int n_tiles, int splits,
                                                     float* __restrict__ part) {
  constexpr int ROWB = CBK * 2;
  constexpr int SLAB = (CBM + BN) * ROWB;
  constexpr int GA = CBM / 64;   // 1 KB A-DMAs per wave per slab (16 rows of 64 B each)
  constexpr int GW = BN / 64;    // ... weights
  constexpr int DPS = GA + GW;
  constexpr int MI = CBM / 64, NI = BN / 64;  // 32-row MFMA blocks per wave (activations, weights)
  static_assert((CNS - 1) * DPS < 64, "DMA wait count must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char smem[CNS * SLAB];

  int bid = wg_x();
  bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);  // a contiguous run of tiles per XCD
  if (bid >= n_tiles * splits) return;
  const int ks = bid / n_tiles;
  bid -= ks * n_tiles;
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int m0 = tm * CBM, n0 = tn * BN;
  const int HW = a.H * a.W, M = a.T * HW;
  const int Cin = 1 << a.cin_log2, K = 27 * Cin, KT_all = (K + CBK - 1) / CBK;
  const int kt0 = ks * KT_all / splits, KT = (ks + 1) * KT_all / splits - kt0;  // this split's slabs

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  // DMA roles: instruction i of this wave fills slab rows 16 (wave + 4 i) + lane / 4,
  // physical chunk lane & 3, which holds logical chunk (lane & 3) ^ cswz(row)
  int pt[GA], ph[GA], pw[GA], ca[GA];
#pragma unroll
  for (int i = 0; i < GA; ++i) {
    const int r = 16 * (wave + 4 * i) + (lane >> 2);
    const int m = min(m0 + r, M - 1);
    pt[i] = m / HW;
    ph[i] = (m - pt[i] * HW) / a.W;
    pw[i] = m - pt[i] * HW - ph[i] * a.W;
    ca[i] = (lane & 3) ^ cswz(r);
  }
  const f16_t* wr[GW];
  int cw[GW];
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int r = 16 * (wave + 4 * i) + (lane >> 2);
    wr[i] = a.w + (int64_t)min(n0 + r, a.cout - 1) * K;
    cw[i] = (lane & 3) ^ cswz(r);
  }
  // the source of this lane's chunk of activation row i in the slab at k0
  auto a_src = [&](int i, int k0) -> const f16_t* {
    const int k = k0 + 8 * ca[i];
    if (k >= K) return a.zero;
    const int tap = k >> a.cin_log2, c = k & (Cin - 1);
    const int dt = tap / 9, dh = (tap / 3) % 3, dw = tap % 3;
    const int t = max(pt[i] + dt - 2, 0), h = ph[i] + dh - 1, w = pw[i] + dw - 1;
    if (h < 0 || h >= a.H || w < 0 || w >= a.W) return a.zero;
    return a.in + ((int64_t)(t * a.H + h) * a.W + w) * Cin + c;
  };
  auto dma_slab = [&](int buf, int kt) {
    char* sb = smem + buf * SLAB;
    const int k0 = (kt0 + min(kt, KT - 1)) * CBK;
#pragma unroll
    for (int i = 0; i < GA; ++i) dma16(a_src(i, k0), sb + (wave + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int k = k0 + 8 * cw[i];
      dma16(wr[i] + (k < K ? k : 0), sb + CBM * ROWB + (wave + 4 * i) * 1024);  // past K: A is zero there
    }
  };

  f32x16 acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // slab kt lives in buffer kt % CNS; slabs 0 .. CNS-2 are fetched up front
#pragma unroll
  for (int s = 0; s < CNS - 1; ++s) dma_slab(s, s);
  const int arow = wm * (CBM / 2) + lr, wrow = CBM + wn * (BN / 2) + lr;
  for (int kt = 0; kt < KT; ++kt) {
    wait_vm<(CNS - 2) * DPS>();  // this wave's DMAs of slab kt have landed
    barrier();                   // everyone's have, and slab kt - 1's buffer is read out
    dma_slab((kt + CNS - 1) % CNS, kt + CNS - 1);
    const char* sb = smem + (kt % CNS) * SLAB;
#pragma unroll
    for (int kk = 0; kk < CBK / 16; ++kk) {
      f16x8 af[MI], wf[NI];
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const int r = arow + 32 * j;
        af[j] = *reinterpret_cast<const f16x8*>(sb + r * ROWB + (((2 * kk + lh) ^ cswz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = wrow + 32 * i;
        wf[i] = *reinterpret_cast<const f16x8*>(sb + r * ROWB + (((2 * kk + lh) ^ cswz(r - CBM)) << 4));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  }
  wait_vm<0>();
  mfma_drain(acc[NI - 1][MI - 1]);

  // epilogue: lane (lr, lh) of block (i, j) holds output channels
  // n0 + wn BN/2 + 32 i + 8 g + 4 lh + e (e = 0..3) of position m0 + wm CBM/2 + 32 j + lr
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int m = m0 + wm * (CBM / 2) + 32 * j + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / 2) + 32 * i + 8 * g + 4 * lh;
        if (n >= a.cout) continue;
        const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if constexpr (EPI == CONV_PART) {
          const f32x4 y = {v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(part + ((int64_t)ks * M + m) * a.cout + n) = y;
        } else {
          store4<EPI>(a, m, n, v);
        }
      }
  }
}

// Halo-tiled form for frames whose width is a multiple of 32 and inputs of at
// least 32 channels. A tile is 4 output rows x 32 columns of one frame. Per
// 32-channel chunk of the input, the tile's whole receptive field -- 3 frames
// (causal, clamped at frame 0) x 6 rows x 34 columns, zero outside the frame --
// is DMA'd to LDS once (HALO_ROWS rows of 64 bytes), and the 27 taps read
// their A fragments from it at shifted rows: per chunk 40 KB of input cross
// L2 -> LDS instead of the 221 KB of a DMA per tap. K runs as (chunk, tap
// group of one time and row offset: 3 column taps); each group's weights (3 x
// BN rows x 32 channels) come through a 3-deep ring. The halo has one buffer,
// refilled between chunks: the stall is covered by a second workgroup on the
// CU, which the 76 KB footprint (BN = 64) allows. Used where the tiles fill
// half the chip or more (the wide layers of stages 1 and 2 and the output
// convolution of a slice); the other layers keep the per-tap kernel above.
// HC = 32 (4 rows) or 16 (8 rows: a 32-position MFMA block is then two image
// rows) columns per tile; the halo buffer (40 KB) holds either receptive field.
constexpr int HALO_DMA = 10;                        // 1 KB DMAs per wave per halo (40 x 16 rows)
constexpr int HALO_BYTES = 4 * HALO_DMA * 1024;     // 40 KB
constexpr int HNS = 3;                              // weight-group ring depth
template <int HC>
struct HaloShape {
  static constexpr int HR = 128 / HC;                       // output rows per tile
  static constexpr int H = HR + 2, W = HC + 2;              // halo positions per frame
  static constexpr int ROWS = 3 * H * W;                    // 612 (HC 32) or 540 (HC 16)
};

template <int BN>
constexpr int halo_smem() { return HALO_BYTES + HNS * 3 * BN * 64; }

// EPI == CONV_PART: split K by input chunks; workgroup split ks multiplies
// chunks [ks nch / splits, (ks + 1) nch / splits) and writes raw F32 sums to
// part[ks][m][n]
template <int BN, int HC, int EPI>
__global__ __launch_bounds__(256, ((halo_smem<BN>() <= 80 * 1024) ? 2 : 1))
void conv3d_halo_kernel(ConvArgs a, int tiles_m, int n_tiles, int splits, float* __restrict__ part) {
  using HS = HaloShape<HC>;
  constexpr int HR = HS::HR, HALO_H = HS::H, HALO_W = HS::W, HALO_ROWS = HS::ROWS;
  constexpr int WG_BYTES = 3 * BN * 64;       // one tap group's weights: [3 column taps][BN][32 channels]
  constexpr int DPS = 3 * BN / 16 / 4;        // weight DMAs per wave per group
  constexpr int NI = BN / 64;                 // 32-channel MFMA blocks per wave
  static_assert((HNS - 1) * DPS < 64, "DMA wait count must fit vmcnt");
  static_assert(HALO_ROWS <= 4 * HALO_DMA * 16, "halo DMAs must cover the halo");
  static_assert(HC == 16 || HC == 32, "16 or 32 columns per tile");
  __shared__ __attribute__((aligned(1024))) char smem[halo_smem<BN>()];
  char* const hbuf = smem;                  // the halo
  char* const wbuf = smem + HALO_BYTES;     // HNS weight groups

  int bid = wg_x();
  bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);  // a contiguous run of tiles per XCD
  if (bid >= n_tiles * splits) return;
  const int ks = bid / n_tiles;
  bid -= ks * n_tiles;
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int wtiles = a.W / HC, htiles = (a.H + HR - 1) / HR;
  const int wb = tm % wtiles, hb = (tm / wtiles) % htiles, t0 = tm / (wtiles * htiles);
  const int h0 = hb * HR, w0 = wb * HC, n0 = tn * BN;
  const int Cin = 1 << a.cin_log2, K = 27 * Cin, nch = Cin >> 5;
  const int c0 = ks * nch / splits, KT = ((ks + 1) * nch / splits - c0) * 9;  // this split's chunks x 9 groups

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  // halo DMA d of this wave fills halo rows 16 (wave + 4 d) + lane / 4, physical
  // chunk lane & 3 (logical chunk (lane & 3) ^ cswz(row)); its source position
  // is fixed per tile, the chunk's channels move with the input chunk
  // (rows outside the frame, and the padding rows past the halo, read the zero row)
  const f16_t* hsrc[HALO_DMA];
  int hstep[HALO_DMA];  // 32 (channels per chunk) for a real source, 0 for the zero row
#pragma unroll
  for (int d = 0; d < HALO_DMA; ++d) {
    const int r = 16 * (wave + 4 * d) + (lane >> 2);
    const int lc = (lane & 3) ^ cswz(r);
    hsrc[d] = a.zero + 8 * lc;
    hstep[d] = 0;
    if (r < HALO_ROWS) {
      const int dt = r / (HALO_H * HALO_W), rem = r - dt * (HALO_H * HALO_W);
      const int hh = rem / HALO_W, ww = rem - hh * HALO_W;
      const int t = max(t0 + dt - 2, 0), h = h0 + hh - 1, w = w0 + ww - 1;
      if (h >= 0 && h < a.H && w >= 0 && w < a.W) {
        hsrc[d] = a.in + ((int64_t)(t * a.H + h) * a.W + w) * Cin + 8 * lc;
        hstep[d] = 32;
      }
    }
  }
  // weight DMA d fills group rows 16 (wave + 4 d) + lane / 4 = column tap dw, channel row n
  const f16_t* wsrc[DPS];
#pragma unroll
  for (int d = 0; d < DPS; ++d) {
    const int r = 16 * (wave + 4 * d) + (lane >> 2);
    const int dw = r / BN, n = r - dw * BN;
    const int lc = (lane & 3) ^ cswz(r);
    wsrc[d] = a.w + (int64_t)min(n0 + n, a.cout - 1) * K + dw * Cin + 8 * lc;
  }
  auto halo_dma = [&](int cc) {
#pragma unroll
    for (int d = 0; d < HALO_DMA; ++d) dma16(hsrc[d] + hstep[d] * cc, hbuf + (wave + 4 * d) * 1024);
  };
  auto w_dma = [&](int buf, int it) {
    const int cc = c0 + it / 9, g = it % 9;  // group g = 3 dt + dh: taps 3 g + dw
#pragma unroll
    for (int d = 0; d < DPS; ++d) dma16(wsrc[d] + 3 * g * Cin + 32 * cc, wbuf + buf * WG_BYTES + (wave + 4 * d) * 1024);
  };

  f32x16 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  halo_dma(c0);
  w_dma(0, 0);
  w_dma(1, min(1, KT - 1));
  for (int it = 0; it < KT; ++it) {
    // this wave's DMAs of group it have landed (and every older one: the first
    // chunk's halo); the next group's may still be in flight
    wait_vm<(HNS - 2) * DPS>();
    barrier();  // everyone's have, and the buffer of group it - 1 is read out
    w_dma((it + 2) % HNS, min(it + 2, KT - 1));
    const int cc = c0 + it / 9, g = it % 9, dt = g / 3, dh = g - 3 * dt;
    if (g == 0 && cc > c0) {  // every wave is past chunk cc - 1: refill the halo
      halo_dma(cc);
      wait_vm<0>();
      barrier();
    }
    const char* hb_ = hbuf;
    const char* wb_ = wbuf + (it % HNS) * WG_BYTES;
    f16x8 af[3][2][2], wf[3][2][NI];
#pragma unroll
    for (int dw = 0; dw < 3; ++dw)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // position 32 (2 wm + j) + lr of the tile: row p / HC, column p % HC
          const int p = 32 * (2 * wm + j) + lr;
          const int r = (dt * HALO_H + p / HC + dh) * HALO_W + p % HC + dw;
          af[dw][kq][j] = *reinterpret_cast<const f16x8*>(hb_ + r * 64 + (((2 * kq + lh) ^ cswz(r)) << 4));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = dw * BN + wn * (BN / 2) + 32 * i + lr;
          wf[dw][kq][i] = *reinterpret_cast<const f16x8*>(wb_ + r * 64 + (((2 * kq + lh) ^ cswz(r)) << 4));
        }
      }
#pragma unroll
    for (int dw = 0; dw < 3; ++dw)
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[dw][kq][i], af[dw][kq][j], acc[i][j], 0, 0, 0);
  }
  wait_vm<0>();
  mfma_drain(acc[NI - 1][1]);

  // epilogue: lane (lr, lh) of block (i, j) holds channels n0 + wn BN/2 + 32 i + 8 g + 4 lh + e
  // of tile position p = 32 (2 wm + j) + lr: frame t0, row h0 + p / HC, column w0 + p % HC
  const int M = a.T * a.H * a.W;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = 32 * (2 * wm + j) + lr;
    const int h = h0 + p / HC;
    if (h >= a.H) continue;
    const int m = (t0 * a.H + h) * a.W + w0 + p % HC;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / 2) + 32 * i + 8 * g + 4 * lh;
        if (n >= a.cout) continue;
        const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if constexpr (EPI == CONV_PART) {
          *reinterpret_cast<f32x4*>(part + ((int64_t)ks * M + m) * a.cout + n) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          store4<EPI>(a, m, n, v);
        }
      }
  }
}

// The split-K convolution's finish: the parts of 4 consecutive channels added
// in index order, then the layer's rounding and store (store4).
template <int EPI>
__global__ __launch_bounds__(256) void conv_reduce_kernel(ConvArgs a, const float* __restrict__ part, int splits) {
  const int64_t M = (int64_t)a.T * a.H * a.W;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= M * (a.cout / 4)) return;
  const int64_t m = q / (a.cout / 4);
  const int n = (int)(q - m * (a.cout / 4)) * 4;
  f32x4 sum = *reinterpret_cast<const f32x4*>(part + m * a.cout + n);
  for (int k = 1; k < splits; ++k) sum = sum + *reinterpret_cast<const f32x4*>(part + (k * M + m) * a.cout + n);
  const float v[4] = {sum[0], sum[1], sum[2], sum[3]};
  store4<EPI>(a, (int)m, n, v);
}

// RMS norm over the C channels of each position (F32 sums), gain, SiLU, F16
// store. C / 8 threads per position, 8 channels (16 bytes) each.
__global__ __launch_bounds__(256) void norm_silu_kernel(const f16_t* __restrict__ x, const float* __restrict__ g,
                                                        f16_t* __restrict__ y, int64_t M, int C, float eps) {
  const int tpp = C >> 3;
  const int64_t p = ((int64_t)blockIdx.x * 256 + threadIdx.x) / tpp;
  const int c = (threadIdx.x % tpp) * 8;
  const bool on = p < M;
  f16x8 v = {};
  if (on) v = *reinterpret_cast<const f16x8*>(x + p * C + c);
  float f[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)v[e];
    ss += f[e] * f[e];
  }
  for (int o = 1; o < tpp; o <<= 1) ss += __shfl_xor(ss, o, 64);
  if (!on) return;
  const float rs = rsqrtf(ss / (float)C + eps);
  f16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float z = f[e] * rs * g[c + e];
    out[e] = (f16_t)(z / (1.f + __expf(-z)));
  }
  *reinterpret_cast<f16x8*>(y + p * C + c) = out;
}

// latent [C][F][H][W] float32 -> channels-last F16 [F][H][W][C]; the first
// 128 threads also clear the decoder's zero row
__global__ __launch_bounds__(256) void latent_f16_kernel(const float* __restrict__ lat, int C, int64_t FHW,
                                                         f16_t* __restrict__ out, f16_t* __restrict__ zero) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < 128) zero[i] = (f16_t)0.f;
  if (i >= (int64_t)C * FHW) return;
  const int64_t pos = i / C;
  const int c = (int)(i - pos * C);
  out[i] = (f16_t)lat[(int64_t)c * FHW + pos];
}

template <int BN, int HC>
hipError_t launch_halo(int epi, const ConvArgs& a, int splits, float* part, hipStream_t s) {
  const int tiles_m = a.T * ((a.H + HaloShape<HC>::HR - 1) / HaloShape<HC>::HR) * (a.W / HC);
  const int tiles = tiles_m * ((a.cout + BN - 1) / BN);
  const dim3 grid((tiles * splits + 7) / 8 * 8), block(256);
#define FH_HALO(E) launch_timed(conv3d_halo_kernel<BN, HC, E>, grid, block, s, a, tiles_m, tiles, splits, part)
  if (splits > 1) {
    FH_HALO(CONV_PART);
    const int64_t M = (int64_t)a.T * a.H * a.W;
    const dim3 rgrid((unsigned)((M * (a.cout / 4) + 255) / 256));
    switch (epi) {
      case CONV_PLAIN: launch_timed(conv_reduce_kernel<CONV_PLAIN>, rgrid, block, s, a, part, splits); break;
      case CONV_RES: launch_timed(conv_reduce_kernel<CONV_RES>, rgrid, block, s, a, part, splits); break;
      case CONV_UP: launch_timed(conv_reduce_kernel<CONV_UP>, rgrid, block, s, a, part, splits); break;
      case CONV_FRAMES: launch_timed(conv_reduce_kernel<CONV_FRAMES>, rgrid, block, s, a, part, splits); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case CONV_PLAIN: FH_HALO(CONV_PLAIN); break;
    case CONV_RES: FH_HALO(CONV_RES); break;
    case CONV_UP: FH_HALO(CONV_UP); break;
    case CONV_FRAMES: FH_HALO(CONV_FRAMES); break;
    default: return hipErrorInvalidValue;
  }
#undef FH_HALO
  return hipGetLastError();
}

template <int BN>
hipError_t launch_conv(int epi, const ConvArgs& a, int splits, float* part, hipStream_t s) {
  const int64_t M = (int64_t)a.T * a.H * a.W;
  const int tiles_m = (int)((M + CBM - 1) / CBM);
  const int tiles = tiles_m * ((a.cout + BN - 1) / BN);
  const dim3 grid((tiles * splits + 7) / 8 * 8), block(256);
  if (splits > 1) {
    launch_timed(conv3d_kernel<BN, CONV_PART>, grid, block, s, a, tiles_m, tiles, splits, part);
    const dim3 rgrid((unsigned)((M * (a.cout / 4) + 255) / 256));
    switch (epi) {
      case CONV_PLAIN: launch_timed(conv_reduce_kernel<CONV_PLAIN>, rgrid, block, s, a, part, splits); break;
      case CONV_RES: launch_timed(conv_reduce_kernel<CONV_RES>, rgrid, block, s, a, part, splits); break;
      case CONV_UP: launch_timed(conv_reduce_kernel<CONV_UP>, rgrid, block, s, a, part, splits); break;
      case CONV_FRAMES: launch_timed(conv_reduce_kernel<CONV_FRAMES>, rgrid, block, s, a, part, splits); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case CONV_PLAIN: launch_timed(conv3d_kernel<BN, CONV_PLAIN>, grid, block, s, a, tiles_m, tiles, 1, part); break;
    case CONV_RES: launch_timed(conv3d_kernel<BN, CONV_RES>, grid, block, s, a, tiles_m, tiles, 1, part); break;
    case CONV_UP: launch_timed(conv3d_kernel<BN, CONV_UP>, grid, block, s, a, tiles_m, tiles, 1, part); break;
    case CONV_FRAMES: launch_timed(conv3d_kernel<BN, CONV_FRAMES>, grid, block, s, a, tiles_m, tiles, 1, part); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int conv_splits(int64_t M, int cin, int cout) {
  // split K where the output tiles cannot fill the chip: up to 256 workgroups,
  // at least 8 slabs of 32 per split
  const int bn = cout >= 128 ? 128 : 64;
  const int64_t tiles = ((M + CBM - 1) / CBM) * ((cout + bn - 1) / bn);
  const int kt = (27 * cin + CBK - 1) / CBK;
  if (tiles >= 128 || kt < 16) return 1;
  int sp = (int)(256 / tiles);
  sp = sp < kt / 8 ? sp : kt / 8;
  return sp < 1 ? 1 : sp;
}

// Which kernel a convolution takes. The halo-tiled one where the frames are a
// whole number of 32- (else 16-) column tiles wide and the input has 32
// channels or more: alone where its tiles fill half the chip, else split over
// input chunks if that brings 128 workgroups or more; otherwise the per-tap
// kernel with its own K split.
struct ConvPlan {
  int halo_hc;  // 32 or 16: halo-tiled with that many columns per tile; 0: per-tap kernel
  int splits;
};
ConvPlan conv_plan(int T, int H, int W, int cin_log2, int cout) {
  if (cin_log2 >= 5) {
    const int hc = W % 32 == 0 ? 32 : W % 16 == 0 ? 16 : 0;
    if (hc) {
      const int hr = 128 / hc;
      const int64_t tiles = (int64_t)T * ((H + hr - 1) / hr) * (W / hc) * ((cout + 63) / 64);
      if (tiles >= 128) return {hc, 1};
      const int64_t sp = std::min<int64_t>(1 << (cin_log2 - 5), 256 / tiles);
      if (sp >= 2 && tiles * sp >= 128) return {hc, (int)sp};
    }
  }
  return {0, conv_splits((int64_t)T * H * W, 1 << cin_log2, cout)};
}

size_t conv_part_elems(int T, int H, int W, int cin, int cout) {
  int cl = 0;
  while ((1 << cl) < cin) ++cl;
  const ConvPlan pl = conv_plan(T, H, W, cl, cout);
  return pl.splits > 1 ? (size_t)pl.splits * T * H * W * cout : 0;
}

hipError_t conv3d_f16(int epi, const ConvArgs& a, float* part, size_t part_elems, hipStream_t s) {
  const int64_t M = (int64_t)a.T * a.H * a.W;
  if (M <= 0) return hipSuccess;
  if (M > (1 << 30) || a.cin_log2 < 3 || a.cin_log2 > 10 || a.cout % 16 || !a.in || !a.w || !a.bias || !a.zero)
    return hipErrorInvalidValue;
  if ((epi == CONV_PLAIN || epi == CONV_RES || epi == CONV_UP) && !a.out) return hipErrorInvalidValue;
  if (epi == CONV_RES && !a.res) return hipErrorInvalidValue;
  if (epi == CONV_UP && (a.cout % 32)) return hipErrorInvalidValue;  // 8 sub-positions x a multiple of 4 channels
  if (epi == CONV_FRAMES && (!a.frames || a.cout % 16)) return hipErrorInvalidValue;
  const ConvPlan pl = conv_plan(a.T, a.H, a.W, a.cin_log2, a.cout);
  const int splits = pl.splits;
  if (splits > 1 && (!part || part_elems < (size_t)splits * M * a.cout)) return hipErrorInvalidValue;
  if (pl.halo_hc == 32) return launch_halo<64, 32>(epi, a, splits, part, s);
  if (pl.halo_hc == 16) return launch_halo<64, 16>(epi, a, splits, part, s);
  // 128 output channels per tile where there are that many, else 64
  return a.cout >= 128 ? launch_conv<128>(epi, a, splits, part, s) : launch_conv<64>(epi, a, splits, part, s);
}

hipError_t norm_silu_f16(const _Float16* x, const float* g, _Float16* y, int64_t M, int C, float eps, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (C < 8 || C > 512 || (C & (C - 1))) return hipErrorInvalidValue;
  const int64_t threads = M * (C / 8);
  launch_timed(norm_silu_kernel, (unsigned)((threads + 255) / 256), 256, s, x, g, y, M, C, eps);
  return hipGetLastError();
}

hipError_t latent_to_f16(const float* lat, int C, int64_t FHW, _Float16* out, _Float16* zero, hipStream_t s) {
  const int64_t n = (int64_t)C * FHW;
  const int64_t total = n > 128 ? n : 128;
  launch_timed(latent_f16_kernel, (unsigned)((total + 255) / 256), 256, s, lat, C, FHW, out, zero);
  return hipGetLastError();
}

hipError_t set_wg_reverse_vae(int r) { return set_wg_reverse(r); }

}  // namespace fh
