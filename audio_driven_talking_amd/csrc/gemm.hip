// bf16 GEMM on gfx950 MFMA: C[M,N] = A[M,K] * W[N,K]^T with fp32 accumulation
// and fused epilogues (bias, tanh-GELU, gated / plain fp32 residual, split
// row-major / transposed store).
//
// Both operands are K-contiguous (activations [tokens, K], weights [out, in]).
// The MFMA is issued as W-fragment x A-fragment, so each lane of a 32x32
// result holds 4 consecutive output columns of one row.
//
// Workgroup tile BM x BN (BM, BN multiples of 64), K-slabs of BK = 32 or 64,
// 256 threads = 4 waves in 2x2, each wave (BM/2) x (BN/2) of MFMA 32x32x16
// blocks; or (KW = 2) two such groups of 4 waves, each taking half of every
// slab's k-steps, which puts two waves on each SIMD (one wave alone cannot
// issue LDS fragment reads fast enough to feed a 64 x 64 wave tile) and adds
// the groups' sums through LDS before the epilogue. Operand slabs go global
// -> LDS directly (global_load_lds_dwordx4: each wave instruction fills 1 KB
// of whole rows), NS slabs deep, one barrier per slab. A slab's fragments are read into registers during the previous
// slab's MFMAs, and the DMA and LDS-read instructions are spread between the
// MFMAs, so neither the address unit nor the LDS stalls the matrix core in
// bursts. The 16-byte chunks of an LDS row are XOR-swizzled so that the
// fragment reads of 16 consecutive rows fall in 16 distinct bank slots.
// The epilogue stages each 32-row block of results in LDS and writes global
// memory in whole row segments.
// Tile order is XCD-aware: the grid is padded to a multiple of the 8 XCDs and
// each XCD gets a contiguous run of tiles, M fastest, so the tiles sharing a
// weight slab share an L2.
// Other forms of the same kernel: split K (f32 parts per K range), K ranges
// multiplied separately and stored side by side (one product per attention
// head), weights chosen per group of rows (one weight matrix per latent
// frame), and a launch over a table of weight pointers (one product per DiT
// block). An MX-FP8 form on the block-scaled MFMA follows below.
#include <cxxabi.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "fh_common.h"

#include "fh_kernels.h"

namespace fh {

namespace {
thread_local LaunchEvents t_launch_ev;

// a GEMM launch: through hipExtLaunchKernelGGL with the armed events, if any
template <typename Kern, typename... Args>
void launch_gemm(Kern kern, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  launch_timed(kern, grid, block, s, args...);
}
}  // namespace

LaunchEvents& armed_launch_events() { return t_launch_ev; }

void arm_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_launch_ev.start = start;
  t_launch_ev.stop = stop;
  t_launch_ev.used = false;
}

bool launch_events_used() {
  const bool u = t_launch_ev.used;
  t_launch_ev = LaunchEvents();
  return u;
}

bool trace_on() {
  static const bool on = [] {
    const char* v = getenv("FH_TRACE");
    return v && v[0] == '1' && v[1] == 0;
  }();
  return on;
}

void trace_line(const void* kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const std::string& args) {
  const char* mangled = hipKernelNameRefByPtr(kern, s);
  int st = -1;
  char* name = mangled ? abi::__cxa_demangle(mangled, nullptr, nullptr, &st) : nullptr;
  std::string n = st == 0 && name ? name : mangled ? mangled : "?";
  free(name);
  // keep the name and template arguments: drop a return type, the namespaces and the parameter types
  if (n.compare(0, 5, "void ") == 0) n.erase(0, 5);
  for (const char* ns : {"(anonymous namespace)::", "fh::"})
    for (size_t at; (at = n.find(ns)) != std::string::npos;) n.erase(at, strlen(ns));
  const size_t paren = n.find('(');
  if (paren != std::string::npos) n.resize(paren);
  fprintf(stderr, "fh launch %s grid %ux%ux%u block %ux%ux%u lds %zu stream %p (%s)\n", n.c_str(), grid.x, grid.y,
          grid.z, block.x, block.y, block.z, lds, (void*)s, args.c_str());
  fflush(stderr);
}
namespace {

constexpr int KALIGN = 64;  // K must be a multiple of this (either slab depth divides it)

// Epilogue staging. After the main loop each wave owns the 32-row blocks of
// its (BM/2) x C sub-tile, C = BN/2 columns. A block goes through the wave's
// own LDS region so that global memory is written (and, for the residual
// forms, read) in whole contiguous row segments instead of one 16-byte piece
// of each of 32 rows per instruction. Row pitches carry 16 bytes of padding
// against LDS bank conflicts.
template <int C>
struct Stage {
  static constexpr int PB = 2 * C + 16;  // bf16 block [32][C]
  static constexpr int PF = 4 * C + 16;  // f32 block [32][C]
  static constexpr int PT = 64 + 16;     // bf16 transposed block [C][32]
  static constexpr int BYTES = (32 * PF > C * PT ? 32 * PF : C * PT);
};

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// The epilogue of a BM x BN tile whose MFMA 32x32 results sit in acc: result
// (i, j) of a wave holds row m = m0 + wm*BM/2 + j*32 + lr and columns
// n = n0 + wn*BN/2 + i*32 + 8g + 4lh + {0..3} in acc[i][j][4g .. 4g+3]. The
// slab buffers must be free (smem reused for staging).
template <int EPI, int BM, int BN, int WN = 2>
__device__ __forceinline__ void store_tile(f32x16 (&acc)[BN / (32 * WN)][BM / 64], char* smem, const EpiArgs& ep,
                                           int M, int N, int m0, int n0, int wm, int wn, int wave, int lane,
                                           int ks) {
  constexpr int MI = BM / 64, NI = BN / (32 * WN), C = BN / WN;
  using ST = Stage<C>;
  const int lr = lane & 31, lh = lane >> 5;
  char* st = smem + wave * ST::BYTES;
  const int nw = n0 + wn * C;  // first column of this wave's sub-tile
  // the transposed form applies to a whole sub-tile (split is a multiple of BN)
  const bool transposed = (EPI == EPI_SPLIT_T || EPI == EPI_SPLIT_T_MX) && nw >= ep.split;
  // residual forms with few values per lane: every x value this lane will update
  // is requested before the first block is staged, so the reads' latency is paid
  // once rather than once per 32-row block
  constexpr int ITS = 32 * C / 4 / 64;
  constexpr bool XPRE = (EPI == EPI_GATED_RES || EPI == EPI_RES) && MI * ITS <= 8;
  f32x4 xv[XPRE ? MI : 1][XPRE ? ITS : 1];
  if constexpr (XPRE) {
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int it = 0; it < ITS; ++it) {
        const int c = it * 64 + lane, row = c / (C / 4), c4 = (c % (C / 4)) * 4;
        const int m = m0 + wm * (BM / 2) + j * 32 + row;
        if (m < M) xv[j][it] = *reinterpret_cast<const f32x4*>(ep.x + (int64_t)m * ep.ldx + nw + c4);
      }
  }
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int mb = m0 + wm * (BM / 2) + j * 32;  // first row of the block
    if (mb >= M) break;
    if constexpr (EPI == EPI_GATED_RES || EPI == EPI_RES || EPI == EPI_PARTIAL) {
      // raw f32 sums -> LDS; then by rows: x[m, n..n+3] += (sum + bias) * gate,
      // or (split K) the sums alone into this split's part
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          *reinterpret_cast<f32x4*>(st + lr * ST::PF + (i * 32 + 8 * g + 4 * lh) * 4) = v;
        }
      lds_fence();
#pragma unroll
      for (int it = 0; it < 32 * C / 4 / 64; ++it) {
        const int c = it * 64 + lane, row = c / (C / 4), c4 = (c % (C / 4)) * 4;
        const int m = mb + row, n = nw + c4;
        if (m < M && EPI == EPI_PARTIAL) {
          *reinterpret_cast<f32x4*>(ep.part + ((int64_t)ks * M + m) * N + n) =
              *reinterpret_cast<const f32x4*>(st + row * ST::PF + c4 * 4);
        } else if (m < M) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * ST::PF + c4 * 4);
          const f32x4 b = *reinterpret_cast<const f32x4*>(ep.bias + n);
          f32x4 u = v + b;
          if constexpr (EPI == EPI_GATED_RES) {
            const f32x4 gt = *reinterpret_cast<const f32x4*>(ep.gate_tab + n);
            const f32x4 ge = *reinterpret_cast<const f32x4*>(ep.gate_e0 + (int64_t)(m / ep.rows_per_lane) * ep.gate_stride + n);
            u = u * (gt + ge);
          }
          f32x4* xp = reinterpret_cast<f32x4*>(ep.x + (int64_t)m * ep.ldx + n);
          if constexpr (XPRE) *xp = xv[j][it] + u;
          else *xp = *xp + u;
        }
      }
      lds_fence();
    } else if constexpr (EPI == EPI_GELU_MX) {
      // raw f32 sums -> LDS; then per lane one 32-column block of a row: bias,
      // GELU, MX-FP8 quantisation, 32 code bytes and the block's scale byte
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          *reinterpret_cast<f32x4*>(st + lr * ST::PF + (i * 32 + 8 * g + 4 * lh) * 4) = v;
        }
      lds_fence();
      constexpr int CB = C / 32, NB = 32 * CB;  // 32-column blocks per row, per 32-row block
#pragma unroll
      for (int it = 0; it < (NB + 63) / 64; ++it) {
        const int blk = it * 64 + lane, row = blk / CB, cb = blk % CB;
        const int m = mb + row, n = nw + 32 * cb;
        if (blk < NB && m < M) {
          float y[32];
          float amax = 0.f;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(st + row * ST::PF + (32 * cb + 4 * t) * 4);
            const f32x4 b = *reinterpret_cast<const f32x4*>(ep.bias + n + 4 * t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              y[4 * t + e] = gelu_tanh(v[e] + b[e]);
              amax = fmaxf(amax, fabsf(y[4 * t + e]));
            }
          }
          const int ex = mx_shared_exp(amax);
          const float inv = mx_inv_scale(ex);
          u32x4 w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x2 a = pack8_e4m3(y + 16 * h, inv), c = pack8_e4m3(y + 16 * h + 8, inv);
            w[h] = u32x4{a.x, a.y, c.x, c.y};
          }
          u32x4* op = reinterpret_cast<u32x4*>(ep.out_q + (int64_t)m * ep.ldq + n);
          op[0] = w[0];
          op[1] = w[1];
          reinterpret_cast<uint8_t*>(ep.q_scale)[((int64_t)(n / 64) * M + m) * 2 + ((n / 32) & 1)] =
              (uint8_t)(ex + 127);
        }
      }
      lds_fence();
    } else if (EPI == EPI_SPLIT_T_MX && transposed) {
      // values as MX-FP8 along the tokens: f32 sums -> LDS [32 rows][C]; then
      // one lane per column: bias, the column's 32-token block maximum, 32
      // codes into out_q[lane][column][token] and the block's scale byte
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          *reinterpret_cast<f32x4*>(st + lr * ST::PF + (i * 32 + 8 * g + 4 * lh) * 4) = v;
        }
      lds_fence();
      const int bl = mb / ep.rows_per_lane, t0 = mb - bl * ep.rows_per_lane;  // a block never spans lanes
#pragma unroll
      for (int cc = 0; cc < C / 64; ++cc) {
        const int col = cc * 64 + lane, n = nw + col;
        const float bias = ep.bias[n];
        float y[32];
        float amax = 0.f;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          // rows past M repeat row M-1: they are not stored, and a copy cannot raise the maximum
          const int rr = mb + r < M ? r : M - 1 - mb;
          y[r] = *reinterpret_cast<const float*>(st + rr * ST::PF + col * 4) + bias;
          amax = fmaxf(amax, fabsf(y[r]));
        }
        const int ex = mx_shared_exp(amax);
        const float inv = mx_inv_scale(ex);
        u32x4 w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2 a = pack8_e4m3(y + 16 * h, inv), b = pack8_e4m3(y + 16 * h + 8, inv);
          w[h] = u32x4{a.x, a.y, b.x, b.y};
        }
        const int64_t vrow = (int64_t)bl * ep.t_cols + (n - ep.split);
        u32x4* op = reinterpret_cast<u32x4*>(ep.out_q + vrow * ep.rows_per_lane + t0);
        op[0] = w[0];
        op[1] = w[1];
        // scales [lane][rows / 64][t_cols] as byte pairs (32-row blocks 2s, 2s+1)
        ep.q_scale_b[(((int64_t)bl * (ep.rows_per_lane / 64) + t0 / 64) * ep.t_cols + (n - ep.split)) * 2 +
                     ((t0 / 32) & 1)] = (uint8_t)(ex + 127);
      }
      lds_fence();
    } else {
      if (!transposed) {
        // (sum + bias [, GELU]) as bf16 -> LDS; then 16-byte pieces of rows
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = nw + i * 32 + 8 * g + 4 * lh;
            const float4 b = *reinterpret_cast<const float4*>(ep.bias + n);
            float c0 = acc[i][j][4 * g] + b.x, c1 = acc[i][j][4 * g + 1] + b.y;
            float c2 = acc[i][j][4 * g + 2] + b.z, c3 = acc[i][j][4 * g + 3] + b.w;
            if constexpr (EPI == EPI_GELU_BF16) {
              c0 = gelu_tanh(c0); c1 = gelu_tanh(c1); c2 = gelu_tanh(c2); c3 = gelu_tanh(c3);
            }
            const u32x2 w = {pack2bf(c0, c1), pack2bf(c2, c3)};
            *reinterpret_cast<u32x2*>(st + lr * ST::PB + (i * 32 + 8 * g + 4 * lh) * 2) = w;
          }
        lds_fence();
#pragma unroll
        for (int it = 0; it < 32 * C / 8 / 64; ++it) {
          const int c = it * 64 + lane, row = c / (C / 8), c8 = (c % (C / 8)) * 8;
          const int m = mb + row;
          const u32x4 w = *reinterpret_cast<const u32x4*>(st + row * ST::PB + c8 * 2);
          if (m < M) *reinterpret_cast<u32x4*>(ep.out_bf + (int64_t)m * ep.ldo + nw + c8) = w;
          if constexpr (EPI == EPI_BF16_SSQ) {
            // squares of the stored values, summed over the C / 8 lanes of the row
            float q = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
              q += lo * lo + hi * hi;
            }
#pragma unroll
            for (int o = 1; o < C / 8; o <<= 1) q += __shfl_xor(q, o, 64);
            if (m < M && c8 == 0) ep.ssq[(int64_t)m * (N / C) + nw / C] = q;
          }
        }
        lds_fence();
      } else {
        // (sum + bias) as bf16, transposed -> LDS [C][32]; then 8 consecutive
        // tokens of one output column per 16-byte piece
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int nl = i * 32 + 8 * g + 4 * lh;
            const float4 b = ep.bias ? *reinterpret_cast<const float4*>(ep.bias + nw + nl) : make_float4(0.f, 0.f, 0.f, 0.f);
            bf16_t* sp = reinterpret_cast<bf16_t*>(st + nl * ST::PT) + lr;
            sp[0] = f2bf(acc[i][j][4 * g] + b.x);
            sp[ST::PT / 2] = f2bf(acc[i][j][4 * g + 1] + b.y);
            sp[ST::PT] = f2bf(acc[i][j][4 * g + 2] + b.z);
            sp[3 * ST::PT / 2] = f2bf(acc[i][j][4 * g + 3] + b.w);
          }
        lds_fence();
        // transposed rows of pitch ldt; a head-split product (split index ks) starts at column ks rows_per_lane
        const int ldt = ep.ldt ? ep.ldt : ep.rows_per_lane;
#pragma unroll
        for (int it = 0; it < C * 4 / 64; ++it) {
          const int c = it * 64 + lane, nl = c / 4, t8 = (c % 4) * 8;
          const int m = mb + t8;  // 8 rows, never across a lane: rows_per_lane % 8 == 0
          if (m < M) {
            const int bl = m / ep.rows_per_lane, t = m - bl * ep.rows_per_lane;
            bf16_t* o = ep.out_t + ((int64_t)bl * ep.t_cols + (nw + nl - ep.split)) * ldt +
                        (int64_t)ks * ep.rows_per_lane + t;
            *reinterpret_cast<u32x4*>(o) = *reinterpret_cast<const u32x4*>(st + nl * ST::PT + t8 * 2);
          }
        }
        lds_fence();
      }
    }
  }
}

// The prefetch wave of a PF launch: it takes the same workgroup barriers as
// the compute waves (the prologue's, one per slab, the one after the loop and,
// with two wave groups, the hand-over's) and between them issues its share of
// the 1 KB pieces of ep.pf into a scratch KB of LDS, spread evenly over slabs
// KT/8 .. 3KT/4: after the tiles' own first fetches from HBM, and early enough
// to land before the tiles end. It never waits on its own loads before a
// barrier (at most 48 in flight), so it cannot hold the others back.
template <int KW>
__device__ __forceinline__ void prefetch_wave(const Prefetch& pf, char* lds, int64_t wg, int64_t n_wg, int KT,
                                              int lane) {
  const int64_t n0 = pf.kb(0), n1 = pf.kb(1), n = n0 + n1 + pf.kb(2);
  const int64_t mine = wg < n ? (n - 1 - wg) / n_wg + 1 : 0;  // pieces wg, wg + n_wg, ...
  int64_t i = 0;
  auto issue_to = [&](int64_t end) {
    for (; i < end; ++i) {
      const int64_t j = wg + i * n_wg;
      const char* src = j < n0        ? static_cast<const char*>(pf.p[0]) + (j << 10)
                        : j < n0 + n1 ? static_cast<const char*>(pf.p[1]) + ((j - n0) << 10)
                                      : static_cast<const char*>(pf.p[2]) + ((j - n0 - n1) << 10);
      wait_vm<48>();
      dma16(src + 16 * lane, lds);
    }
  };
  const int k0 = KT / 8, k1 = max(k0 + 1, 3 * KT / 4);
  barrier();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt >= k0) issue_to(mine * min(kt - k0 + 1, k1 - k0) / (k1 - k0));
    barrier();
  }
  barrier();
  if (KW == 2) barrier();
  wait_vm<0>();
}

// WN = 4: one group of 2 x 4 waves (two waves per SIMD, each a (BM/2) x (BN/4)
// sub-tile); the slab's 1 KB DMA groups may then not divide evenly among the
// waves, and a wave's wait counts follow its own share.
template <int EPI, int BM, int BN, int BK, int NS, int KW, bool BATCH, bool PF, int WN = 2>
__global__ __launch_bounds__(128 * WN * KW + (PF ? 64 : 0),
                             (KW == 1 && WN == 2 && !PF && smem_bytes<BM, BN, BK, NS>() <= 80 * 1024) ? 2 : 1)
void gemm_bf16_nt(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ W, int ldw,
                  int M, int N, int K, int tiles_m, int tiles, int splits, EpiArgs ep) {
  constexpr int NG = 2 * WN;           // waves per group (2 x WN)
  constexpr int NW = NG * KW;          // waves: KW groups, group g takes k-steps g KK/KW ..
  constexpr int ROWB = BK * 2;         // bytes per LDS row of a slab
  constexpr int CH = BK / 8;           // 16-byte chunks per row
  constexpr int RG = 64 / CH;          // rows per 1 KB DMA group
  constexpr int MI = BM / 64;          // 32-row activation blocks per wave
  constexpr int NI = BN / (32 * WN);   // 32-row weight blocks per wave
  constexpr int TA = BM / RG, TW = BN / RG;   // 1 KB DMA groups per slab, activations / weights
  constexpr int GA = (TA + NW - 1) / NW;      // ... at most per wave
  constexpr int GW = (TW + NW - 1) / NW;
  constexpr int SLAB = (BM + BN) * ROWB;
  static_assert(BM % 64 == 0 && BN % (32 * WN) == 0 && TA * RG == BM && TW * RG == BN, "tile shape");
  static_assert(WN == 2 || (WN == 4 && KW == 1 && !BATCH), "2 x 4 waves: one group, plain launches");
  static_assert(WN == 4 || (GA * NW == TA && GW * NW == TW), "2 x 2 waves share the DMA groups evenly");
  static_assert(GW * NW == TW && (GA * NW == TA || GA * NW - TA < NW), "at most one group fewer per wave");
  static_assert(KW == 1 || KW == 2, "one or two wave groups along K");
  static_assert(NS >= 2 && (NS - 1) * (GA + GW) < 64, "DMA wait count must fit vmcnt");
  static_assert(!PF || !BATCH, "prefetch only in plain launches");
  static_assert(!PF || WN == 2, "prefetch wave only beside 2 x 2 waves");
  __shared__ __attribute__((aligned(1024))) char smem[NS * SLAB + (PF ? 1024 : 0)];

  int bid = wg_x();
  const int per_xcd = gridDim.x >> 3;
  bid = (bid & 7) * per_xcd + (bid >> 3);
  if (bid >= tiles * splits * (BATCH ? ep.batch_n : 1)) return;
  if constexpr (BATCH) {
    // entry e of the table: its weights and bias, its rows of A and its output
    const int e = bid / (tiles * splits);
    bid -= e * tiles * splits;
    const BatchEntry be = ep.batch[e];
    W = be.W;
    ep.bias = be.bias;
    A += (int64_t)e * ep.batch_a_stride;
    if (ep.out_bf) ep.out_bf += (int64_t)e * ep.batch_out_stride;
    if (ep.out_t) ep.out_t += (int64_t)e * ep.batch_out_stride;
  }
  // split ks of K (splits > 1 only with EPI_PARTIAL) covers columns [ks K/splits, (ks+1) K/splits)
  const int ks = bid / tiles, tile = bid - ks * tiles;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  K /= splits;
  A += (int64_t)ks * K;
  W += (int64_t)ks * K;
  if (ep.w_group_rows) W += (int64_t)(m0 / ep.w_group_rows) * ep.w_group_stride;  // a tile is in one group

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / NG;                    // wave group along K
  const int wm = (wave / WN) & 1, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  // whether this wave takes GA activation DMA groups (wave + NW i < TA), or one fewer
  constexpr bool EVEN = GA * NW == TA;
  const bool a_full = EVEN || wave + NW * (GA - 1) < TA;
  if constexpr (PF) {
    if (wave == NW) {
      prefetch_wave<KW>(ep.pf, smem + NS * SLAB, tm + (int64_t)tiles_m * tn + (int64_t)ks * tiles,
                        (int64_t)tiles * splits, K / BK, lane);
      return;
    }
  }

  // DMA: lane fills LDS row r = RG g + lane/CH, physical chunk lane%CH, which
  // holds logical chunk (lane%CH) ^ swz(r); every wave of both groups takes
  // its share of the slab's 1 KB groups
  const int drow = lane / CH;
  const bf16_t* ga[GA];
  const bf16_t* gw[GW];
#pragma unroll
  for (int i = 0; i < GA; ++i) {
    const int r = RG * (wave + NW * i) + drow;
    ga[i] = A + (int64_t)min(m0 + r, M - 1) * lda + ((lane % CH) ^ swz<BK>(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int r = RG * (wave + NW * i) + drow;
    gw[i] = W + (int64_t)(n0 + r) * ldw + ((lane % CH) ^ swz<BK>(r)) * 8;
  }

  // one DMA instruction d of a slab: d < GA an activation group, else a weight group
  auto dma_one = [&](int d, int buf, int k0) {
    char* sa = smem + buf * SLAB;
    if (d < GA) {
      if (EVEN || d < GA - 1 || a_full) dma16(ga[d] + k0, sa + (wave + NW * d) * 1024);
    } else dma16(gw[d - GA] + k0, sa + BM * ROWB + (wave + NW * (d - GA)) * 1024);
  };

  f32x16 acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragments of a whole slab are held in registers, in two sets: while the
  // MFMAs of slab kt run on one set, the fragments of slab kt + 1 are read
  // into the other. Rows: activations wm*BM/2 + 32 j + lr, weights
  // wn*BN/WN + 32 i + lr; the wave's k-step kk covers the slab's k-columns
  // 16 (kg KK + kk) .. +15 (KK k-steps per wave group).
  constexpr int KK = BK / 16 / KW, P = NI * MI, NR = NI + MI, DPS = GA + GW;
  static_assert(KK * 16 * KW == BK, "slab splits evenly between the wave groups");
  constexpr int SLOTS = KK * P, READS = KK * NR;
  const int xr = swz<BK>(lr);
  const int a_row = (wm * (BM / 2) + lr) * ROWB, w_row = BM * ROWB + (wn * (BN / WN) + lr) * ROWB;
  bf16x8 wf[2][KK][NI], af[2][KK][MI];
  // fragment read r of a slab: k-step r / NR; r % NR < NI a weight block, else activations
  auto read_one = [&](int r, int set, int buf) {
    const int kk = r / NR, q = r % NR;
    const char* sb = smem + buf * SLAB + (((2 * (kg * KK + kk) + lh) ^ xr) * 16);
    if (q < NI) wf[set][kk][q] = *reinterpret_cast<const bf16x8*>(sb + w_row + q * 32 * ROWB);
    else af[set][kk][q - NI] = *reinterpret_cast<const bf16x8*>(sb + a_row + (q - NI) * 32 * ROWB);
  };
  // The slab's MFMAs on register set `set`, with the next slab's fragment
  // reads (read r after MFMA slot r*SLOTS/READS) and this iteration's DMA
  // instructions (d after slot d*SLOTS/DPS) spread between them, so the LDS
  // and the address unit work while the matrix core is busy instead of
  // stalling every wave on a burst of requests.
  auto mma_slab = [&](auto set_c, int rbuf, int dbuf, int dk0) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[set][kk][i], af[set][kk][j], acc[i][j], 0, 0, 0);
          const int slot = kk * P + i * MI + j;
#pragma unroll
          for (int r = 0; r < READS; ++r)
            if (r * SLOTS / READS == slot) read_one(r, set ^ 1, rbuf);
#pragma unroll
          for (int d = 0; d < DPS; ++d)
            if (d * SLOTS / DPS == slot) dma_one(d, dbuf, dk0);
          __builtin_amdgcn_sched_barrier(0);
        }
  };

  // Slab kt lives in buffer kt % NS. Slabs 0 .. NS-1 are fetched up front.
  // Iteration kt waits until slab kt + 1 has landed and every wave holds the
  // fragments of slab kt in registers, then (one barrier) multiplies slab kt
  // while it reads slab kt + 1's fragments and refills buffer kt % NS with
  // slab kt + NS, which then has NS - 1 iterations to land. Slabs past the
  // end re-fetch the last one into buffers nobody reads, which keeps the
  // wait counts uniform.
  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int d = 0; d < DPS; ++d) dma_one(d, s, min(s, KT - 1) * BK);
  // wait until at most n slabs' DMAs of this wave are in flight
  auto wait_slabs = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    if (a_full) wait_vm<n * DPS>();
    else wait_vm<n * (DPS - 1)>();
  };
  wait_slabs(std::integral_constant<int, NS - 1>{});
  barrier();
#pragma unroll
  for (int r = 0; r < READS; ++r) read_one(r, 0, 0);
  auto iteration = [&](int kt, auto set_c) {
    wait_slabs(std::integral_constant<int, NS - 2>{});  // this wave's DMAs of slab kt + 1 have landed
    wait_lgkm0();               // and its fragments of slab kt are in registers
    barrier();                  // so for every wave: slab kt + 1 is in, buffer kt % NS is free
    mma_slab(set_c, (kt + 1) % NS, kt % NS, min(kt + NS, KT - 1) * BK);
  };
  // two slabs per trip so that the register set of each is a constant
  for (int kt = 0; kt < KT; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < KT) iteration(kt + 1, std::integral_constant<int, 1>{});
  }
  wait_vm<0>();

  static_assert(NG * Stage<BN / WN>::BYTES <= NS * SLAB, "epilogue staging must fit the slab buffers");
  wait_lgkm0();
  barrier();  // every wave is done with the slab buffers (its DMAs landed above)
  if constexpr (KW == 2) {
    // group 1 hands its sums to group 0 through LDS past the four epilogue
    // staging regions (lane-contiguous 16-byte pieces), then leaves
    constexpr int RED = (4 * Stage<BN / 2>::BYTES + 255) / 256 * 256;
    static_assert(RED + 4 * P * 16 * 64 * 4 <= NS * SLAB, "hand-over buffer must fit the slab buffers");
    float4* red = reinterpret_cast<float4*>(smem + RED) + (wave & 3) * P * 4 * 64 + lane;
    if (kg) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            red[((i * MI + j) * 4 + q) * 64] =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
    barrier();
    if (kg) return;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = red[((i * MI + j) * 4 + q) * 64];
          acc[i][j][4 * q] += v.x;
          acc[i][j][4 * q + 1] += v.y;
          acc[i][j][4 * q + 2] += v.z;
          acc[i][j][4 * q + 3] += v.w;
        }
  }
  store_tile<EPI, BM, BN, WN>(acc, smem, ep, M, N, m0, n0, wm, wn, wave, lane, ks);
}

// ---------------------------------------------------------------- MX-FP8
// The same pipeline on MX-FP8 operands and the block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3): K-slabs of 64 bytes, each
// one MFMA k-step. A lane of half h holds bytes [16h, 16h + 16) and
// [32 + 16h, 48 + 16h) of its row's 64 (two 16-byte LDS reads), which puts
// bytes 0..15 of both halves in 32-element block 0 and bytes 16..31 in
// block 1; the E8M0 scale of (row, block b) comes from the lane of half b,
// so each lane passes the byte of block h of its row. The slab's scales
// (two bytes per row) travel with it by 4-byte-per-lane DMAs (a lane moves
// the pair of two rows; one instruction covers 128 rows): the activation
// rows' scales first (rounded up to 128 rows), then the weight rows'.
template <int BM>
constexpr int mx_arows() { return (BM + 127) / 128 * 128; }
// SB bytes of K per row and slab (64 or 128: one or two 64-deep MFMA k-steps),
// then the scales of each k-step: (activation rows rounded to 128 + weight rows) u16
template <int BM, int BN, int SB = 64>
constexpr int mx_slab_bytes() { return (BM + BN) * SB + ((mx_arows<BM>() + BN) * 2 * (SB / 64) + 1023) / 1024 * 1024; }

__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }  // 64-byte rows
// 16-byte chunk swizzle of an SB-byte slab row (128-byte rows as the bf16 kernel's 64-deep slabs)
template <int SB>
__device__ __forceinline__ int swz_mx(int row) { return SB == 64 ? swz64(row) : (row >> 1) & 7; }

// WN = 4: 2 x 4 waves (two per SIMD), the activation DMA groups dealt as in
// the bf16 kernel (a wave may take one fewer; its wait counts follow). FFN up
// runs so (32.5 -> 30.3 us at 1280 tokens); the QKV tiles were slower.
// SB = 128: slabs of two 64-byte k-steps (half the slab iterations, barriers and
// waits per FLOP; twice the fragment registers).
template <int EPI, int BM, int BN, int NS, int WN = 2, int SB = 64>
__global__ __launch_bounds__(128 * WN, 1)
void gemm_mx_nt(const uint8_t* __restrict__ A, int lda, const uint16_t* __restrict__ As,
                const uint8_t* __restrict__ W, int ldw, const uint16_t* __restrict__ Ws,
                int M, int N, int K, int tiles_m, int tiles, int splits, EpiArgs ep) {
  constexpr int KK = SB / 64;                 // 64-byte k-steps per slab
  constexpr int ROWB = SB, CH = SB / 16, RG = 1024 / SB;  // bytes per LDS row, 16-byte chunks, rows per 1 KB DMA
  constexpr int NW = 2 * WN;                  // waves, 2 x WN
  constexpr int MI = BM / 64, NI = BN / (32 * WN);
  constexpr int TA = BM / RG, TW = BN / RG;   // 1 KB code DMAs per slab, activations / weights
  constexpr int GA = (TA + NW - 1) / NW, GW = (TW + NW - 1) / NW;  // ... at most per wave
  constexpr int SQA = mx_arows<BM>() / 128, SQ1 = SQA + BN / 128;  // 256-byte scale DMAs per k-step
  constexpr int SQ = KK * SQ1;                       // ... per slab
  constexpr int SPW = (SQ + NW - 1) / NW;            // scale DMAs per wave (the last one repeated)
  constexpr int DPS = GA + GW + SPW;
  constexpr int SCB = (BM + BN) * ROWB;              // scale area of a slab
  constexpr int SCK = (mx_arows<BM>() + BN) * 2;     // scale bytes of one k-step
  constexpr int SLAB = mx_slab_bytes<BM, BN, SB>();
  static_assert(SB == 64 || SB == 128, "slabs of one or two 64-byte k-steps");
  static_assert(TA * RG == BM && TW * RG == BN && BN % 128 == 0 && BN % (32 * WN) == 0, "tile shape");
  static_assert(WN == 2 || WN == 4, "2 x 2 or 2 x 4 waves");
  static_assert(GW * NW == TW && (GA * NW == TA || GA * NW - TA < NW), "at most one group fewer per wave");
  static_assert(NS >= 2 && (NS - 1) * DPS < 64, "DMA wait count must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char smem[NS * SLAB];

  int bid = wg_x();
  const int per_xcd = gridDim.x >> 3;
  bid = (bid & 7) * per_xcd + (bid >> 3);
  if (bid >= tiles * splits) return;
  const int ks = bid / tiles, tile = bid - ks * tiles;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int slabs_all = K / 64;
  K /= splits;
  const int s_base = ks * (K / 64);  // first slab of this split

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  (void)slabs_all;
  // whether this wave takes GA activation DMA groups (wave + NW i < TA), or one fewer
  constexpr bool EVEN = GA * NW == TA;
  const bool a_full = EVEN || wave + NW * (GA - 1) < TA;

  const int drow = lane / CH;
  const uint8_t* ga[GA];
  const uint8_t* gw[GW];
#pragma unroll
  for (int i = 0; i < GA; ++i) {
    const int r = RG * (wave + NW * i) + drow;
    ga[i] = A + (int64_t)min(m0 + r, M - 1) * lda + (int64_t)s_base * 64 + ((lane % CH) ^ swz_mx<SB>(r)) * 16;
  }
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int r = RG * (wave + NW * i) + drow;
    gw[i] = W + (int64_t)(n0 + r) * ldw + (int64_t)s_base * 64 + ((lane % CH) ^ swz_mx<SB>(r)) * 16;
  }
  // scale DMA t of this wave (instruction q2 = SQ1 kk + q: k-step kk of the
  // slab): rows 128 q + 2 lane and the next, of the activations for q < SQA
  // (past M: the last row pair again), else of the weights
  const uint16_t* gs[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    const int q2 = min(wave + NW * t, SQ - 1), kk = q2 / SQ1, q = q2 % SQ1;
    gs[t] = q < SQA ? As + (int64_t)(s_base + kk) * M + min(m0 + 128 * q + 2 * lane, M - 2)
                    : Ws + (int64_t)(s_base + kk) * N + (n0 + 128 * (q - SQA) + 2 * lane);
  }
  auto dma_one = [&](int d, int buf, int slab) {
    char* sb = smem + buf * SLAB;
    if (d < GA) {
      if (EVEN || d < GA - 1 || a_full) dma16(ga[d] + slab * SB, sb + (wave + NW * d) * 1024);
    } else if (d < GA + GW) {
      dma16(gw[d - GA] + slab * SB, sb + BM * ROWB + (wave + NW * (d - GA)) * 1024);
    } else {
      const int t = d - GA - GW, q2 = min(wave + NW * t, SQ - 1), kk = q2 / SQ1, q = q2 % SQ1;
      const int64_t step = q < SQA ? M : N;  // u16 elements per 64-byte k-step in this scale array
      __builtin_amdgcn_global_load_lds((gbl_void*)(gs[t] + (int64_t)slab * KK * step),
                                       (lds_void*)(sb + SCB + kk * SCK + q * 256), 4, 0, 0);
    }
  };

  f32x16 acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  typedef int v8i __attribute__((ext_vector_type(8)));
  constexpr int P = NI * MI, NR = NI + MI;
  const int a_row = wm * (BM / 2) + lr, w_row = BM + wn * (BN / WN) + lr;  // slab rows (W after A)
  v8i wf[2][KK][NI], af[2][KK][MI];
  int wsc[2][KK][NI], asc[2][KK][MI];
  // fragment read r of a slab (and its scale byte): k-step r / NR; r % NR < NI
  // weights, else activations
  auto read_one = [&](int r, int set, int buf) {
    const int kk = r / NR, q = r % NR;
    const char* sb = smem + buf * SLAB;
    const int row = q < NI ? w_row + 32 * q : a_row + 32 * (q - NI);
    const char* rp = sb + row * ROWB;
    const int x = swz_mx<SB>(row);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(rp + (((4 * kk + lh) ^ x) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(rp + (((4 * kk + 2 + lh) ^ x) << 4));
    const v8i f = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const int srow = q < NI ? mx_arows<BM>() + (row - BM) : row;  // row in the scale area
    const int sc = (int)(*reinterpret_cast<const uint16_t*>(sb + SCB + kk * SCK + srow * 2) >> (8 * lh));
    if (q < NI) { wf[set][kk][q] = f; wsc[set][kk][q] = sc; }
    else { af[set][kk][q - NI] = f; asc[set][kk][q - NI] = sc; }
  };
  constexpr int SLOTS = KK * P, READS = KK * NR;
  auto mma_slab = [&](auto set_c, int rbuf, int dbuf, int dslab) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[set][kk][i], af[set][kk][j], acc[i][j], 0,
                                                                      0, 0, wsc[set][kk][i], 0, asc[set][kk][j]);
          const int slot = kk * P + i * MI + j;
#pragma unroll
          for (int r = 0; r < READS; ++r)
            if (r * SLOTS / READS == slot) read_one(r, set ^ 1, rbuf);
#pragma unroll
          for (int d = 0; d < DPS; ++d)
            if (d * SLOTS / DPS == slot) dma_one(d, dbuf, dslab);
          __builtin_amdgcn_sched_barrier(0);
        }
  };

  const int KT = K / SB;
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0)
#pragma unroll
    for (int d = 0; d < DPS; ++d) dma_one(d, s0, min(s0, KT - 1));
  // wait until at most n slabs' DMAs of this wave are in flight
  auto wait_slabs = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    if (a_full) wait_vm<n * DPS>();
    else wait_vm<n * (DPS - 1)>();
  };
  wait_slabs(std::integral_constant<int, NS - 1>{});
  barrier();
#pragma unroll
  for (int r = 0; r < READS; ++r) read_one(r, 0, 0);
  auto iteration = [&](int kt, auto set_c) {
    wait_slabs(std::integral_constant<int, NS - 2>{});  // this wave's DMAs of slab kt + 1 have landed
    wait_lgkm0();               // and its fragments of slab kt are in registers
    barrier();                  // so for every wave: slab kt + 1 is in, buffer kt % NS is free
    mma_slab(set_c, (kt + 1) % NS, kt % NS, min(kt + NS, KT - 1));
  };
  for (int kt = 0; kt < KT; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < KT) iteration(kt + 1, std::integral_constant<int, 1>{});
  }
  wait_vm<0>();
  static_assert(NW * Stage<BN / WN>::BYTES <= NS * SLAB, "epilogue staging must fit the slab buffers");
  wait_lgkm0();
  barrier();
  store_tile<EPI, BM, BN, WN>(acc, smem, ep, M, N, m0, n0, wm, wn, wave, lane, ks);
}

// one thread per 32-element block: codes and the block's scale byte
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T* __restrict__ in, int64_t rows, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  if (b >= rows * nb) return;
  const int64_t row = b / nb;
  const int kb = (int)(b - row * nb);
  const T* p = in + row * K + 32 * kb;
  float y[32];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    if constexpr (sizeof(T) == 4) y[e] = p[e];
    else y[e] = bf2f(p[e]);
    amax = fmaxf(amax, fabsf(y[e]));
  }
  const int ex = mx_shared_exp(amax);
  const float inv = mx_inv_scale(ex);
  u32x4 w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x2 a = pack8_e4m3(y + 16 * h, inv), c = pack8_e4m3(y + 16 * h + 8, inv);
    w[h] = u32x4{a.x, a.y, c.x, c.y};
  }
  u32x4* op = reinterpret_cast<u32x4*>(codes + row * K + 32 * kb);
  op[0] = w[0];
  op[1] = w[1];
  reinterpret_cast<uint8_t*>(scales)[((int64_t)(kb / 2) * rows + row) * 2 + (kb & 1)] = (uint8_t)(ex + 127);
}

template <int BM, int BN, int NS, int WN = 2, int SB = 64>
hipError_t launch_mx(int epi, const uint8_t* A, int lda, const uint16_t* As, const uint8_t* W, int ldw,
                     const uint16_t* Ws, int M, int N, int K, const EpiArgs& ep, hipStream_t s,
                     int splits = 1) {
  if (N % BN || splits < 1 || K % (splits * SB) || lda % 16 || ldw % 16 || M % 2) return hipErrorInvalidValue;
  if (ep.w_group_rows || ep.ldt) return hipErrorInvalidValue;  // bf16 kernel only
  if (splits > 1 && (epi != EPI_PARTIAL || !ep.part || ep.part_elems < (size_t)splits * M * N))
    return hipErrorInvalidValue;
  if (epi == EPI_GELU_MX && (!ep.out_q || !ep.q_scale || ep.ldq % 16)) return hipErrorInvalidValue;
  if ((epi == EPI_SPLIT_T || epi == EPI_SPLIT_T_MX) && (ep.split % BN || ep.rows_per_lane <= 0 || ep.rows_per_lane % 8))
    return hipErrorInvalidValue;
  if (epi == EPI_SPLIT_T_MX && (ep.rows_per_lane % 64 || M % ep.rows_per_lane || !ep.out_q || !ep.q_scale_b ||
                                (BN / WN) % 64))
    return hipErrorInvalidValue;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = tiles_m * (N / BN);
  const dim3 grid((tiles * splits + 7) / 8 * 8), block(128 * WN);
#define FH_MX(E) launch_gemm(gemm_mx_nt<E, BM, BN, NS, WN, SB>, grid, block, s, A, lda, As, W, ldw, Ws, M, N, K, tiles_m, tiles, splits, ep)
  if constexpr (SB != 64) {  // 128-byte slabs: the split-K and QKV products
    if (epi == EPI_PARTIAL) FH_MX(EPI_PARTIAL);
    else if (epi == EPI_SPLIT_T_MX) FH_MX(EPI_SPLIT_T_MX);
    else return hipErrorInvalidValue;
  } else if constexpr (WN == 4) {  // 2 x 4 waves: the FFN up product
    if (epi == EPI_GELU_MX) FH_MX(EPI_GELU_MX);
    else return hipErrorInvalidValue;
  } else {
    switch (epi) {
      case EPI_BF16: FH_MX(EPI_BF16); break;
      case EPI_GELU_MX: FH_MX(EPI_GELU_MX); break;
      case EPI_GATED_RES: FH_MX(EPI_GATED_RES); break;
      case EPI_RES: FH_MX(EPI_RES); break;
      case EPI_PARTIAL: FH_MX(EPI_PARTIAL); break;
      case EPI_SPLIT_T: FH_MX(EPI_SPLIT_T); break;
      case EPI_SPLIT_T_MX: FH_MX(EPI_SPLIT_T_MX); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef FH_MX
  return hipGetLastError();
}

// x[m, n] += gate * (sum_s part[s][m, n] + bias[n]) (gate = 1 without a table),
// the parts added in index order; 4 columns per thread
__global__ __launch_bounds__(256) void residual_from_parts_kernel(float* __restrict__ x, int ldx, PendingRes r,
                                                                  int M, int N) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  f32x4* xp = reinterpret_cast<f32x4*>(x + (int64_t)m * ldx + n);
  *xp = apply_pending(r, *xp, m, n, M, N);
}

template <int BM, int BN, int BK, int NS, int KW = 1, bool BATCH = false, bool PF = false, int WN = 2>
hipError_t launch(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                  const EpiArgs& ep, hipStream_t s, int splits = 1) {
  if (N % BN || splits < 1 || K % (splits * BK)) return hipErrorInvalidValue;
  if (epi == EPI_SPLIT_T && (ep.split % BN || ep.rows_per_lane <= 0 || ep.rows_per_lane % 8))
    return hipErrorInvalidValue;
  if (epi == EPI_SPLIT_T_MX && (ep.split % BN || ep.rows_per_lane <= 0 || ep.rows_per_lane % 64 || M % ep.rows_per_lane ||
                                !ep.out_q || !ep.q_scale_b || (BN / 2) % 64))
    return hipErrorInvalidValue;
  if (epi == EPI_GATED_RES && ep.rows_per_lane <= 0) return hipErrorInvalidValue;
  // splits > 1: K halves summed through f32 parts, or (EPI_SPLIT_T, all columns transposed) one
  // separate product per split placed side by side in rows of pitch ldt
  const bool head_split = epi == EPI_SPLIT_T && ep.split == 0 && ep.ldt >= splits * ep.rows_per_lane;
  if (splits > 1 && !head_split && (epi != EPI_PARTIAL || !ep.part || ep.part_elems < (size_t)splits * M * N))
    return hipErrorInvalidValue;
  if (epi == EPI_SPLIT_T && ep.ldt && (ep.ldt < ep.rows_per_lane || ep.ldt % 8)) return hipErrorInvalidValue;
  if (ep.w_group_rows && (ep.w_group_rows % BM || ep.w_group_stride <= 0)) return hipErrorInvalidValue;
  if (BATCH != (ep.batch != nullptr) || ep.batch_n < 1) return hipErrorInvalidValue;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = tiles_m * (N / BN);
  const int64_t wgs = (int64_t)tiles * splits * ep.batch_n;
  if (wgs > (int64_t)1 << 30) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((wgs + 7) / 8 * 8)), block(128 * WN * KW + (PF ? 64 : 0));
#define FH_GEMM(E) launch_gemm(gemm_bf16_nt<E, BM, BN, BK, NS, KW, BATCH, PF, WN>, grid, block, s, A, lda, W, ldw, M, N, K, tiles_m, tiles, splits, ep)
  if constexpr (WN == 4) {  // 2 x 4 waves
    if (epi == EPI_GELU_BF16) FH_GEMM(EPI_GELU_BF16);
    else if (epi == EPI_SPLIT_T) FH_GEMM(EPI_SPLIT_T);
    else if (epi == EPI_GATED_RES) FH_GEMM(EPI_GATED_RES);
    else if (epi == EPI_RES) FH_GEMM(EPI_RES);
    else if (epi == EPI_BF16) FH_GEMM(EPI_BF16);
    else if (epi == EPI_BF16_SSQ) FH_GEMM(EPI_BF16_SSQ);
    else return hipErrorInvalidValue;
  } else if constexpr (PF) {  // the forms that prefetch: the residual, query and split-K products
    if (!ep.pf.any()) return hipErrorInvalidValue;
    if (epi == EPI_GATED_RES) FH_GEMM(EPI_GATED_RES);
    else if (epi == EPI_RES) FH_GEMM(EPI_RES);
    else if (epi == EPI_BF16_SSQ) FH_GEMM(EPI_BF16_SSQ);
    else if (epi == EPI_PARTIAL) FH_GEMM(EPI_PARTIAL);
    else return hipErrorInvalidValue;
  } else {
    switch (epi) {
      case EPI_BF16: FH_GEMM(EPI_BF16); break;
      case EPI_GELU_BF16: FH_GEMM(EPI_GELU_BF16); break;
      case EPI_GATED_RES: FH_GEMM(EPI_GATED_RES); break;
      case EPI_RES: FH_GEMM(EPI_RES); break;
      case EPI_SPLIT_T: FH_GEMM(EPI_SPLIT_T); break;
      case EPI_SPLIT_T_MX: FH_GEMM(EPI_SPLIT_T_MX); break;
      case EPI_PARTIAL: FH_GEMM(EPI_PARTIAL); break;
      case EPI_BF16_SSQ: FH_GEMM(EPI_BF16_SSQ); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef FH_GEMM
  return hipGetLastError();
}

}  // namespace

// Tile choice from measurements of the slice shapes on MI355X with weights
// cold in HBM (as in a 30-block slice). Big tiles need less L2->LDS traffic
// per FLOP; the counts are chosen so one round of tiles about fills the 256
// CUs (e.g. FFN-up at 1280 tokens: 7 x 35 = 245 tiles of 192 x 256).
int gemm_tile_choice(int M, int N, int K) {
  (void)K;
  if (M <= 256) return 3;                                   // 64x128 k64 s4 (audio K/V)
  if (N % 256 == 0 && N >= 8192) return M <= 1536 ? 0 : 1;  // 192x256 k32 s3 | s4
  if (M <= 1536 && N <= 2048) return 2;                     // 128x64 k64 s4
  return 4;                                                 // 192x128 k64 s3
}

bool gemm_splitk_ok(int M, int N, int K) {
  // residual GEMMs of width <= 2048 with a long K at up to 1536 tokens: 128 x 128
  // tiles over two halves of K fill the chip with less operand traffic per FLOP
  // than 128 x 64 tiles; short K does not pay for the extra pass over the parts
  return M > 0 && M <= 1536 && N % 128 == 0 && N <= 2048 && K >= 4096 && K % 128 == 0;
}

bool gemm_splitk_wide_ok(int M, int N, int K) {
  // 1536 < M <= 3072 (a 768 x 768 slice: 2880 tokens): 192 x 192 tiles over two K halves make
  // 15 x 8 x 2 = 240 workgroups where unsplit 192 x 128 tiles make 180 (at three 1280-token
  // streams the unsplit tiles already make 240, and 256 x 192 halves lost more in the
  // LayerNorm that adds the parts than they gained)
  return M > 1536 && M <= 3072 && N % 192 == 0 && N <= 2048 && K >= 4096 && K % 128 == 0;
}

hipError_t gemm_bf16_splitk(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                            float* part, size_t part_elems, hipStream_t s, const Prefetch& pf) {
  if (lda % 8 || ldw % 8) return hipErrorInvalidValue;
  EpiArgs ep;
  ep.part = part;
  ep.part_elems = part_elems;
  if (gemm_splitk_wide_ok(M, N, K)) return launch<192, 192, 64, 3>(EPI_PARTIAL, A, lda, W, ldw, M, N, K, ep, s, 2);
  if (!gemm_splitk_ok(M, N, K)) return hipErrorInvalidValue;
  ep.pf = pf;
  // two wave groups along K: 2.3 % faster than one group on the FFN down-projection at 1280 tokens
  if (pf.any()) return launch<128, 128, 64, 4, 2, false, true>(EPI_PARTIAL, A, lda, W, ldw, M, N, K, ep, s, 2);
  return launch<128, 128, 64, 4, 2>(EPI_PARTIAL, A, lda, W, ldw, M, N, K, ep, s, 2);
}

hipError_t gemm_bf16_splitk_n(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, int splits,
                              float* part, size_t part_elems, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % 128 || splits < 1 || K % (64 * splits) || lda % 8 || ldw % 8 || !part ||
      part_elems < (size_t)splits * M * N)
    return hipErrorInvalidValue;
  EpiArgs ep;
  ep.part = part;
  ep.part_elems = part_elems;
  return launch<64, 128, 64, 4>(EPI_PARTIAL, A, lda, W, ldw, M, N, K, ep, s, splits);
}

hipError_t gemm_bf16_heads(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, int heads,
                           bf16_t* out, int rows_per_lane, int ldt, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (heads < 1 || K % (64 * heads) || N % 128 || lda % 8 || ldw % 8 || !out || rows_per_lane <= 0 ||
      rows_per_lane % 8 || M % rows_per_lane || ldt < heads * rows_per_lane)
    return hipErrorInvalidValue;
  EpiArgs ep;
  ep.out_t = out;
  ep.split = 0;
  ep.t_cols = N;
  ep.rows_per_lane = rows_per_lane;
  ep.ldt = ldt;
  // two stages when each workgroup has only two 64-deep slabs (K / heads = 128), as in the batched form
  if (K / heads == 128) {
    if (M <= 256) return launch<64, 128, 64, 2>(EPI_SPLIT_T, A, lda, W, ldw, M, N, K, ep, s, heads);
    return launch<128, 64, 64, 2>(EPI_SPLIT_T, A, lda, W, ldw, M, N, K, ep, s, heads);
  }
  if (M <= 256) return launch<64, 128, 64, 4>(EPI_SPLIT_T, A, lda, W, ldw, M, N, K, ep, s, heads);
  return launch<128, 64, 64, 4>(EPI_SPLIT_T, A, lda, W, ldw, M, N, K, ep, s, heads);
}

template <int BM, int BN, int NS>
hipError_t launch_batched(int epi, const bf16_t* A, int lda, int ldw, int M, int N, int K, const EpiArgs& ep,
                          hipStream_t s, int splits) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = tiles_m * (N / BN);
  const int64_t wgs = (int64_t)tiles * splits * ep.batch_n;
  if (N % BN || K % (splits * 64) || wgs > (int64_t)1 << 30) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((wgs + 7) / 8 * 8)), block(256);
  // W comes from the table; the argument only fills the slot
  if (epi == EPI_BF16)
    launch_gemm(gemm_bf16_nt<EPI_BF16, BM, BN, 64, NS, 1, true, false>, grid, block, s, A, lda, (const bf16_t*)nullptr,
                ldw, M, N, K, tiles_m, tiles, splits, ep);
  else
    launch_gemm(gemm_bf16_nt<EPI_SPLIT_T, BM, BN, 64, NS, 1, true, false>, grid, block, s, A, lda, (const bf16_t*)nullptr,
                ldw, M, N, K, tiles_m, tiles, splits, ep);
  return hipGetLastError();
}

hipError_t gemm_bf16_batched(int epi, const bf16_t* A, int lda, int64_t a_stride, const BatchEntry* tab, int nb,
                             int ldw, int M, int N, int K, int heads, const EpiArgs& ep_in, int64_t out_stride,
                             hipStream_t s) {
  if (M <= 0 || nb <= 0) return hipSuccess;
  if (!tab || heads < 1 || lda % 8 || ldw % 8 || K % (64 * heads) || a_stride < 0 || out_stride < 0)
    return hipErrorInvalidValue;
  EpiArgs ep = ep_in;
  ep.batch = tab;
  ep.batch_n = nb;
  ep.batch_a_stride = a_stride;
  ep.batch_out_stride = out_stride;
  if (epi == EPI_BF16) {
    if (heads != 1 || !ep.out_bf || ep.ldo % 8) return hipErrorInvalidValue;
  } else if (epi == EPI_SPLIT_T) {
    if (ep.split != 0 || !ep.out_t || ep.rows_per_lane <= 0 || ep.rows_per_lane % 8 || M % ep.rows_per_lane ||
        ep.ldt < heads * ep.rows_per_lane || ep.ldt % 8 || ep.t_cols != N)
      return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  // a head-split product runs two 64-deep slabs per workgroup: two stages, so nothing is fetched twice
  // and up to three workgroups share a CU
  if (heads > 1 && K / heads == 128) {
    if (M <= 256) return launch_batched<64, 128, 2>(epi, A, lda, ldw, M, N, K, ep, s, heads);
    return launch_batched<128, 64, 2>(epi, A, lda, ldw, M, N, K, ep, s, heads);
  }
  // 128 < M <= 192 (one lane's 160 audio tokens): every row in one tile, so each weight slab
  // crosses L2 -> LDS once instead of once per 64-row tile
  if (M > 128 && M <= 192) return launch_batched<192, 128, 3>(epi, A, lda, ldw, M, N, K, ep, s, heads);
  if (M <= 256) return launch_batched<64, 128, 4>(epi, A, lda, ldw, M, N, K, ep, s, heads);
  return launch_batched<128, 64, 4>(epi, A, lda, ldw, M, N, K, ep, s, heads);
}

namespace {
__global__ void fill_batch_table_kernel(BatchEntry* dst, BatchTableArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) dst[i] = BatchEntry{(const bf16_t*)a.w[i], (const float*)a.b[i], (const float*)a.g[i]};
}
}  // namespace

hipError_t fill_batch_table(BatchEntry* dst, const BatchTableArgs& args, hipStream_t s) {
  if (!dst || args.n < 1 || args.n > MAX_BATCH_TABLE) return hipErrorInvalidValue;
  launch_timed(fill_batch_table_kernel, 1, MAX_BATCH_TABLE, s, dst, args);
  return hipGetLastError();
}

hipError_t gemm_bf16_grouped(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                             int group_rows, int64_t group_stride, const EpiArgs& ep_in, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if ((epi != EPI_RES && epi != EPI_GATED_RES && epi != EPI_BF16) || N % 128 || K % KALIGN || lda % 8 ||
      ldw % 8 || group_rows <= 0 || group_rows % 64 || group_stride <= 0)
    return hipErrorInvalidValue;
  EpiArgs ep = ep_in;
  ep.w_group_rows = group_rows;
  ep.w_group_stride = group_stride;
  // a tile never spans two groups: 128-row tiles where the groups allow, else 64
  if (group_rows % 128 == 0) {
    if (ep.pf.any() && epi != EPI_BF16)
      return launch<128, 64, 64, 4, 1, false, true>(epi, A, lda, W, ldw, M, N, K, ep, s);
    return launch<128, 64, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
  }
  return launch<64, 128, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
}

hipError_t residual_from_parts(float* x, int ldx, const PendingRes& r, int M, int N, hipStream_t s) {
  if (M <= 0 || !r.part) return hipSuccess;
  if (N % 4 || ldx % 4 || r.nparts < 1 || (r.gate_tab && r.rows_per_lane <= 0)) return hipErrorInvalidValue;
  launch_timed(residual_from_parts_kernel, (unsigned)(((int64_t)M * N / 4 + 255) / 256), 256, s, x, ldx, r, M, N);
  return hipGetLastError();
}

int gemm_ssq_groups(int M, int N, int K) {
  // columns per wave of each gemm_tile_choice's tiles: BN / 2, or BN / 4 where 2 x 4 waves run them
  const int c = gemm_tile_choice(M, N, K);
  static const int cols[] = {128, 128, 32, 64, 64};
  return N / (c == 4 && M > 1536 ? 32 : cols[c]);
}

hipError_t gemm_bf16(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                     const EpiArgs& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (epi == EPI_BF16_SSQ && !ep.ssq) return hipErrorInvalidValue;
  if (N % 128 || K % KALIGN || lda % 8 || ldw % 8 || epi == EPI_PARTIAL) return hipErrorInvalidValue;
  switch (gemm_tile_choice(M, N, K)) {
    case 0:
      if (epi == EPI_GELU_BF16) return launch<192, 256, 32, 3, 1, false, false, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
      return launch<192, 256, 32, 3>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case 1:
      if (epi == EPI_GELU_BF16) return launch<192, 256, 32, 4, 1, false, false, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
      return launch<192, 256, 32, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case 2:
      // a fifth wave fits beside these tiles' registers (no spill), so they carry the prefetch
      if (ep.pf.any() && (epi == EPI_GATED_RES || epi == EPI_RES || epi == EPI_BF16_SSQ))
        return launch<128, 64, 64, 4, 1, false, true>(epi, A, lda, W, ldw, M, N, K, ep, s);
      return launch<128, 64, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
    case 3: return launch<64, 128, 64, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
    default:
      if (epi == EPI_SPLIT_T ||
          (M > 1536 && (epi == EPI_GATED_RES || epi == EPI_RES || epi == EPI_BF16 || epi == EPI_BF16_SSQ)))
        return launch<192, 128, 64, 3, 1, false, false, 4>(epi, A, lda, W, ldw, M, N, K, ep, s);
      return launch<192, 128, 64, 3>(epi, A, lda, W, ldw, M, N, K, ep, s);
  }
}

hipError_t gemm_mx(int epi, const uint8_t* A, int lda, const uint16_t* As, const uint8_t* W, int ldw,
                   const uint16_t* Ws, int M, int N, int K, const EpiArgs& ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % 128 || K % 64 || epi == EPI_PARTIAL) return hipErrorInvalidValue;
  // stage counts from a same-process A/B of the FP8 slice (3 beat 4 and 5 here; 4 beat 3, 6 and 8 for split K);
  // 192 x 256 tiles only where they still give most CUs a tile (FFN up: 245 at 1280 tokens; QKV: 126 -> 192 x 128)
  const int64_t tiles_wide = (int64_t)((M + 191) / 192) * (N / 256);
  if (N % 256 == 0 && N >= 4096 && tiles_wide >= 200) {
    if (epi == EPI_GELU_MX) return launch_mx<192, 256, 3, 4>(epi, A, lda, As, W, ldw, Ws, M, N, K, ep, s);
    return launch_mx<192, 256, 3>(epi, A, lda, As, W, ldw, Ws, M, N, K, ep, s);
  }
  // QKV with MX-FP8 values: 128-byte slabs (3 stages) measured faster (22.0 -> 19.1 us at 1280
  // tokens); with bf16 outputs the epilogue sets the time and they do not pay
  if (epi == EPI_SPLIT_T_MX && K % 128 == 0)
    return launch_mx<192, 128, 3, 2, 128>(epi, A, lda, As, W, ldw, Ws, M, N, K, ep, s);
  return launch_mx<192, 128, 5>(epi, A, lda, As, W, ldw, Ws, M, N, K, ep, s);
}

hipError_t gemm_mx_splitk(const uint8_t* A, int lda, const uint16_t* As, const uint8_t* W, int ldw,
                          const uint16_t* Ws, int M, int N, int K, float* part, size_t part_elems,
                          hipStream_t s) {
  if (!gemm_splitk_ok(M, N, K)) return hipErrorInvalidValue;
  EpiArgs ep;
  ep.part = part;
  ep.part_elems = part_elems;
  if (K % 256 == 0) return launch_mx<128, 128, 4, 2, 128>(EPI_PARTIAL, A, lda, As, W, ldw, Ws, M, N, K, ep, s, 2);
  return launch_mx<128, 128, 4>(EPI_PARTIAL, A, lda, As, W, ldw, Ws, M, N, K, ep, s, 2);
}

hipError_t mx_quantize(const float* in_f, const bf16_t* in_b, int64_t rows, int K, uint8_t* codes,
                       uint16_t* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 64 || (!in_f == !in_b) || !codes || !scales) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((rows * (K / 32) + 255) / 256);
  if (in_f) launch_timed(mx_quantize_kernel<float>, grid, 256, s, in_f, rows, K, codes, scales);
  else launch_timed(mx_quantize_kernel<bf16_t>, grid, 256, s, in_b, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t set_wg_reverse_gemm(int r) { return set_wg_reverse(r); }

}  // namespace fh
