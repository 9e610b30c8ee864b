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
// flash_attn: 64 queries per workgroup, the 4 waves split as 2 query groups x
// 2 key halves (so a 1280-token slice gives 240 workgroups per lane); K and
// V^T blocks are DMA'd into XOR-swizzled LDS, double-buffered.
// cross_attn: short key ranges (32 audio tokens per latent frame, or all of
// them), fragments loaded straight from global memory, no LDS.
// cross_probs: the frame-local softmax probabilities alone (the value
// product is folded into the output projection's GEMM).
// flash_attn_mx: the self-attention on MX-FP8 operands (block-scaled MFMA).
#include "fh_common.h"
#include "fh_kernels.h"

namespace fh {
namespace {

constexpr int HD = 128;
constexpr int KB = 64;

__device__ __forceinline__ bf16x8 load_v_frag(const bf16_t* p) {
  // keys {0..3} and {8..11} relative to p (see the key permutation above)
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  const u32x4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 p_frag(const f32x16& st, int u) {
  const u32x4 w = {pack2bf(st[8 * u], st[8 * u + 1]), pack2bf(st[8 * u + 2], st[8 * u + 3]),
                   pack2bf(st[8 * u + 4], st[8 * u + 5]), pack2bf(st[8 * u + 6], st[8 * u + 7])};
  return __builtin_bit_cast(bf16x8, w);
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

// Self-attention workgroup: 64 queries of one (lane, head); wave w takes
// query group w & 1 (32 queries) and key half w >> 1. Each step stages one
// 64-key block of each half (K [64 x 128] and V^T [128 x 64], bf16) into LDS
// by DMA, XOR-swizzled on 16-byte chunks, double-buffered; the two halves'
// online-softmax states are merged through LDS at the end.
//
// Key order: the MFMA row i of a 32-key tile reads key kperm(i) (bits 2 and 3
// swapped), so the 8 scores a lane holds for one 16-key k-step are 8
// contiguous keys; the matching V^T fragment is then one 16-byte LDS read.
// Rescaling is lazy: the reference maximum moves only when a block's maximum
// exceeds it by more than 2^TAU, so P stays <= 2^TAU (exact in the final
// normalisation) and the accumulators are rarely touched by VALU.
constexpr int AQ = 64;                 // queries per workgroup
constexpr int KBLK = KB * HD * 2;      // bytes of one K (or V^T) block
constexpr int ASTAGE = 4 * KBLK;       // K and V^T of both halves
constexpr float TAU = 8.f;

__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// Chunk swizzles. gfx950 serves 16-byte LDS reads in 16-lane groups over a
// 256-byte bank window: the 16 K rows (256 B each) a fragment read touches
// take 16 distinct chunks via row & 15; the 16 V^T rows (128 B, two per
// window) take 8 distinct chunks per row parity via (row >> 1) & 7.
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256, 1) void flash_attn_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ k, int ldk,
    const bf16_t* __restrict__ vt, bf16_t* __restrict__ o, int ldo, int N, int D,
    float scale_log2, int n_qt, int n_heads, int n_wg) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * ASTAGE];
  // workgroups are dealt round-robin to the 8 XCDs; give each XCD a run of
  // consecutive (query tile fastest) workgroups so the query tiles of a head
  // share one L2 copy of its keys and values
  const unsigned bx = wg_x();
  const int wg = (bx & 7) * (gridDim.x >> 3) + (bx >> 3);
  if (wg >= n_wg) return;
  const int qt = wg % n_qt, h = (wg / n_qt) % n_heads, b = wg / (n_qt * n_heads);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave & 1, kh = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = qt * AQ + qg * 32;

  bf16x8 qf[8];
  {
    const int qrow = min(q0 + lr, N - 1);
    const bf16_t* qp = q + ((int64_t)b * N + qrow) * ldq + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  const int nkb = (N + KB - 1) / KB;
  const int nh0 = (nkb + 1) / 2;  // key blocks of half 0; half 1 has nkb - nh0

  // DMA roles of this lane: K rows 4g + lane/16 (16 chunks of 16 B per row),
  // V^T rows 8g + lane/8 (8 chunks per row), g = 4 wave + i
  const bf16_t* kbase = k + (int64_t)b * N * ldk + h * HD;
  const bf16_t* vbase = vt + ((int64_t)b * D + h * HD) * N;
  // DMA instruction d < 16 of a step: key half d >> 3, group i = (d >> 1) & 3,
  // the K rows (d even) or the V^T rows (d odd)
  auto issue_one = [&](int d, int buf, int j) {
    char* st = smem + buf * ASTAGE;
    const int c = d >> 3, i = (d >> 1) & 3;
    const int kb = min(c == 0 ? j : nh0 + j, nkb - 1);
    const int g = 4 * wave + i;
    if ((d & 1) == 0) {
      const int krow = 4 * g + (lane >> 4);
      const int kch = (lane & 15) ^ kswz(krow);
      const int key = min(kb * KB + krow, N - 1);
      dma16(kbase + (int64_t)key * ldk + kch * 8, st + c * 2 * KBLK + g * 1024);
    } else {
      const int vrow = 8 * g + (lane >> 3);
      const int vch = (lane & 7) ^ vswz(vrow);
      const int vkey = min(kb * KB + vch * 8, N - 8);
      dma16(vbase + (int64_t)vrow * N + vkey, st + c * 2 * KBLK + KBLK + g * 1024);
    }
  };
  auto issue = [&](int buf, int j) {
#pragma unroll
    for (int d = 0; d < 16; ++d) issue_one(d, buf, j);
  };

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int krow_l = kperm(lr);
  const int kx = kswz(krow_l), vx = vswz(lr);

  // Every step refills the other buffer (past the last step with the clamped
  // last block, which nobody reads); the DMA instructions go out one after
  // each score MFMA, so their address arithmetic runs under the matrix core.
  issue(0, 0);
  for (int j = 0; j < nh0; ++j) {
    wait_vm<0>();
    barrier();
    const int kb = kh == 0 ? j : nh0 + j;
    if (kb >= nkb) {
      issue((j + 1) & 1, j + 1);
      continue;
    }
    const char* kp = smem + (j & 1) * ASTAGE + kh * 2 * KBLK;
    const char* vp = kp + KBLK;

    f32x16 st[2];
    bf16x8 kf[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
      const char* krow = kp + (32 * t + krow_l) * (HD * 2);
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[t][s] = *reinterpret_cast<const bf16x8*>(krow + (((2 * s + lh) ^ kx) << 4));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][s], qf[s], st[t], 0, 0, 0);
        issue_one(2 * s + t, (j + 1) & 1, j + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    // st[t][r] is the score of key kb*64 + 32t + 16(r>>3) + 8lh + (r&7)
    if ((kb + 1) * KB > N) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * KB + 32 * t + 16 * (r >> 3) + 8 * lh + (r & 7) >= N) st[t][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    if (__any(mx > m_run + TAU)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[t][r], scale_log2, -m_run));
        st[t][r] = p;
        ps += p;
      }
    l_run += ps;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pf = p_frag(st[t], u);
        const int c = 4 * t + 2 * u + lh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vp + (32 * dt + lr) * (KB * 2) + ((c ^ vx) << 4));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[dt], 0, 0, 0);
        }
      }
  }
  l_run += __shfl_xor(l_run, 32, 64);

  // merge the key halves: wave (qg, 1) hands (m, l, acc) to wave (qg, 0)
  wait_vm<0>();
  barrier();
  float* mg = reinterpret_cast<float*>(smem) + qg * (66 * 64);
  if (kh == 1) {
    mg[lane] = m_run;
    mg[64 + lane] = l_run;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mg[(2 + dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = mg[lane], l1 = mg[64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float inv = 1.f / (l_run * a0 + l1 * a1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = acc[dt][r] * a0 + mg[(2 + dt * 16 + r) * 64 + lane] * a1;
    if (q0 + lr < N) store_o(o + ((int64_t)b * N + q0 + lr) * ldo + h * HD, acc, inv, lh);
  }
}

// MX-FP8 self-attention (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3).
// Same workgroup shape as flash_attn (64 queries, 2 query groups x 2 key
// halves, 64-key blocks, double-buffered DMA). Differences:
//  * S^T = K Q^T takes two scaled MFMAs per 32-key tile (k-steps of 64 dims);
//    each operand lane-half h supplies bytes [16h, 16h+16) of both 32-wide
//    blocks of a k-step and the E8M0 scale of its row's block h;
//  * MFMA row i of a tile reads key kperm_mx(i) = 16 bit2(i) + 4 (i >> 3) +
//    (i & 3), so lane-half h ends up holding the scores of keys 16h .. 16h+15
//    in order -- exactly the bytes the P^T operand of the next product wants;
//  * the probabilities are quantised per query and 32-key tile (block
//    maximum with one exchange between the lane halves) and O^T = V^T P^T is
//    one scaled MFMA per 32 output dims;
//  * the running sum l is of the unquantised probabilities.
// LDS of a key half per stage: K codes [64 keys][128 B] (chunk swizzle
// kswz_mx), V^T codes [128 dims][64 B] (vswz_mx), K scales [64][4 B], V
// scales [128][2 B].
__device__ __forceinline__ int kperm_mx(int i) { return ((i & 4) << 2) | ((i >> 3) << 2) | (i & 3); }
// 16-lane fragment reads touch rows {0..7, 16..23} or {8..15, 24..31} of a tile
// (two 128-byte rows per bank window): these take 16 distinct 16-byte slots
__device__ __forceinline__ int kswz_mx(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }
__device__ __forceinline__ int vswz_mx(int r) { return (r >> 2) & 3; }
constexpr int MXK_CODES = 64 * HD;                 // 8 KB
constexpr int MXV_CODES = HD * 64;                 // 8 KB
constexpr int MX_HALF = MXK_CODES + MXV_CODES + 1024;  // + K and V scales (256 B each), 1 KB aligned
constexpr int MX_STAGE = 2 * MX_HALF;
typedef int v8i_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i_t frag_mx(const char* row, int c_lo, int c_hi) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(row + (c_lo << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(row + (c_hi << 4));
  return v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ __launch_bounds__(256, 1) void flash_attn_mx_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ qs, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ ks, int ldq, const uint8_t* __restrict__ vt, const uint8_t* __restrict__ vts,
    bf16_t* __restrict__ o, int ldo, int N, int D, float scale_log2, int n_qt, int n_heads, int n_wg) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * MX_STAGE];
  const unsigned bx = wg_x();
  const int wg = (bx & 7) * (gridDim.x >> 3) + (bx >> 3);
  if (wg >= n_wg) return;
  const int qt = wg % n_qt, h = (wg / n_qt) % n_heads, b = wg / (n_qt * n_heads);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave & 1, kh = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = qt * AQ + qg * 32;
  const int lds_q = ldq / 32;  // scale bytes per row

  // this lane's query: k-step s holds bytes [64s + 16lh, +16) and [64s + 32 + 16lh, +16)
  v8i_t qf[2];
  int qsc[2];
  {
    const int qrow = min(q0 + lr, N - 1);
    const uint8_t* qp = q + ((int64_t)b * N + qrow) * ldq + h * HD;
    const uint8_t* sp = qs + ((int64_t)b * N + qrow) * lds_q + h * 4;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      qf[s2] = frag_mx(reinterpret_cast<const char*>(qp + 64 * s2), lh, 2 + lh);
      qsc[s2] = sp[2 * s2 + lh];
    }
  }

  const int nkb = N / 64;
  const int nh0 = (nkb + 1) / 2;
  const uint8_t* kbase = k + (int64_t)b * N * ldq + h * HD;
  const uint8_t* ksbase = ks + (int64_t)b * N * lds_q + h * 4;
  const uint8_t* vbase = vt + ((int64_t)b * D + h * HD) * N;
  const uint8_t* vsbase = vts + (int64_t)b * (N / 64) * D * 2 + h * HD * 2;
  // DMA d = 9 wave + i of 36 per stage: half d / 18; e = d % 18: K code rows 8e..8e+7 (e < 8),
  // V^T code rows 16(e-8)..+15 (e < 16), the K scales (e = 16), the V scales (e = 17)
  auto issue = [&](int buf, int j) {
    char* stg = smem + buf * MX_STAGE;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int d = 9 * wave + i, c = d / 18, e = d % 18;
      const int kb = min(c == 0 ? j : nh0 + j, nkb - 1);
      char* hp = stg + c * MX_HALF;
      if (e < 8) {
        const int row = 8 * e + (lane >> 3);
        const int ch = (lane & 7) ^ kswz_mx(row);
        dma16(kbase + (int64_t)(kb * 64 + row) * ldq + ch * 16, hp + e * 1024);
      } else if (e < 16) {
        const int row = 16 * (e - 8) + (lane >> 2);
        const int ch = (lane & 3) ^ vswz_mx(row);
        dma16(vbase + (int64_t)row * N + kb * 64 + ch * 16, hp + MXK_CODES + (e - 8) * 1024);
      } else if (e == 16) {
        __builtin_amdgcn_global_load_lds((gbl_void*)(ksbase + (int64_t)(kb * 64 + lane) * lds_q),
                                         (lds_void*)(hp + MXK_CODES + MXV_CODES), 4, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds((gbl_void*)(vsbase + ((int64_t)kb * D + 2 * lane) * 2),
                                         (lds_void*)(hp + MXK_CODES + MXV_CODES + 256), 4, 0, 0);
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int krow_l = kperm_mx(lr);

  issue(0, 0);
  for (int j = 0; j < nh0; ++j) {
    wait_vm<0>();
    barrier();
    if (j + 1 < nh0) issue((j + 1) & 1, j + 1);
    const int kb = kh == 0 ? j : nh0 + j;
    if (kb >= nkb) continue;
    const char* hp = smem + (j & 1) * MX_STAGE + kh * MX_HALF;
    const char* kp = hp;
    const char* vp = hp + MXK_CODES;
    const uint8_t* ksp = reinterpret_cast<const uint8_t*>(hp + MXK_CODES + MXV_CODES);
    const uint8_t* vsp = ksp + 256;

    f32x16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
      const int row = 32 * t + krow_l;
      const int x = kswz_mx(row);
      const char* rp = kp + row * HD;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const v8i_t kf = frag_mx(rp, (4 * s2 + lh) ^ x, (4 * s2 + 2 + lh) ^ x);
        const int ksc = ksp[row * 4 + 2 * s2 + lh];
        st[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[s2], st[t], 0, 0, 0, ksc, 0, qsc[s2]);
      }
    }
    // st[t][r] is the score of key kb*64 + 32t + 16lh + r
    if ((kb + 1) * 64 > N) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 64 + 32 * t + 16 * lh + r >= N) st[t][r] = -INFINITY;
    }
    // per-tile score maxima (the row maximum is their maximum): the largest
    // probability of a tile is exp2 of its largest scaled score, exp2 being monotonic
    float tmax[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float v = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, st[t][r]);
      tmax[t] = fmaxf(v, __shfl_xor(v, 32, 64)) * scale_log2;  // the tile's 32 keys of this query
    }
    const float mx = fmaxf(tmax[0], tmax[1]);
    if (__any(mx > m_run + TAU)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    int pex[2];
    u32x4 pc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pex[t] = mx_shared_exp(__builtin_amdgcn_exp2f(tmax[t] - m_run));
      // exp2(y - e) = p * 2^-e: the codes' operands straight from the exponential;
      // they stay below 512 (p <= 2^(e+9)), only the e4m3 range needs a clamp
      const float moff = -m_run - (float)pex[t];
      float q[16], qs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = __builtin_amdgcn_exp2f(fmaf(st[t][r], scale_log2, moff));
        qs += v;
        q[r] = fminf(v, 448.f);
      }
      l_run += qs * __uint_as_float((uint32_t)(pex[t] + 127) << 23);  // sum of p = 2^e * sum of p 2^-e
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // four codes per word: low half, then high half
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * e], q[4 * e + 1], 0, false);
        w[e] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * e + 2], q[4 * e + 3], lo, true);
      }
      pc[t] = w;
    }
    const v8i_t pf = {(int)pc[0].x, (int)pc[0].y, (int)pc[0].z, (int)pc[0].w,
                      (int)pc[1].x, (int)pc[1].y, (int)pc[1].z, (int)pc[1].w};
    const int psc = (lh ? pex[1] : pex[0]) + 127;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int row = 32 * dt + lr;
      const int x = vswz_mx(row);
      const v8i_t vf = frag_mx(vp + row * 64, lh ^ x, (2 + lh) ^ x);
      const int vsc = vsp[row * 2 + lh];
      acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, acc[dt], 0, 0, 0, vsc, 0, psc);
    }
  }
  l_run += __shfl_xor(l_run, 32, 64);

  // merge the key halves as flash_attn does
  barrier();
  float* mg = reinterpret_cast<float*>(smem) + qg * (66 * 64);
  if (kh == 1) {
    mg[lane] = m_run;
    mg[64 + lane] = l_run;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mg[(2 + dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = mg[lane], l1 = mg[64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float inv = 1.f / (l_run * a0 + l1 * a1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = acc[dt][r] * a0 + mg[(2 + dt * 16 + r) * 64 + lane] * a1;
    if (q0 + lr < N) store_o(o + ((int64_t)b * N + q0 + lr) * ldo + h * HD, acc, inv, lh);
  }
}

// Cross-attention: one wave (workgroup) per 32 queries of one (lane, head),
// so a slice launches one wave per 32 tokens and head across the whole chip.
// Keys are the audio tokens of the query's latent frame (or all of them);
// each key block's K and V fragments are requested together, straight from
// global memory (they are small and shared through L2), before the scores.
constexpr int MAXG = 64;  // most column groups of the query sums of squares

// The MFMA B-operand fragments of 32 query rows q0 .. q0+31 of head h (row
// lr of lane half lh: dims 16 s + 8 lh .. +7 in qf[s]), with the query
// RMSNorm over the full width applied when ssq is given. q_request issues
// every load (the fragments, the row's column-group sums, the head's gains)
// and q_finish waits for them and applies the norm, so a caller can put its
// own independent loads in between.
struct QReq {
  bf16x8 qf[8];
  f32x4 part[MAXG / 4];
  f32x4 gv[16];
};

__device__ __forceinline__ void q_request(QReq& r, const bf16_t* __restrict__ q, int ldq, int b, int h, int q0,
                                          int N, const float* __restrict__ ssq, int groups,
                                          const float* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int qrow = min(q0 + lr, N - 1);
  const bf16_t* qp = q + ((int64_t)b * N + qrow) * ldq + h * HD + 8 * lh;
#pragma unroll
  for (int s = 0; s < 8; ++s) r.qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  if (ssq) {
    // all of the row's group sums requested at once (16-byte loads)
    const f32x4* sp = reinterpret_cast<const f32x4*>(ssq + ((int64_t)b * N + qrow) * groups);
#pragma unroll
    for (int p = 0; p < MAXG / 4; ++p)
      if (4 * p < groups) r.part[p] = sp[p];
    const float* gp = g + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.gv[2 * s] = *reinterpret_cast<const f32x4*>(gp + 16 * s);
      r.gv[2 * s + 1] = *reinterpret_cast<const f32x4*>(gp + 16 * s + 4);
    }
  }
}

__device__ __forceinline__ void q_finish(QReq& r, bf16x8 (&qf)[8], int D, const float* __restrict__ ssq,
                                         int groups, float eps) {
  if (ssq) {
    // RMSNorm of the query row over the full width: the group sums added in order
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < MAXG / 4; ++p)
      if (4 * p < groups) ss = (((ss + r.part[p][0]) + r.part[p][1]) + r.part[p][2]) + r.part[p][3];
    const float rs = rsqrtf(ss / (float)D + eps);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f32x4 g0 = r.gv[2 * s], g1 = r.gv[2 * s + 1];
      const u32x4 raw = __builtin_bit_cast(u32x4, r.qf[s]);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        w[e] = pack2bf(__uint_as_float(raw[e] << 16) * rs * g0[2 * e],
                       __uint_as_float(raw[e] & 0xffff0000u) * rs * g0[2 * e + 1]);
        w[e + 2] = pack2bf(__uint_as_float(raw[e + 2] << 16) * rs * g1[2 * e],
                           __uint_as_float(raw[e + 2] & 0xffff0000u) * rs * g1[2 * e + 1]);
      }
      r.qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = r.qf[s];
}

__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[8], const bf16_t* __restrict__ q, int ldq, int b, int h,
                                             int q0, int N, int D, const float* __restrict__ ssq, int groups,
                                             const float* __restrict__ g, float eps) {
  QReq r;
  q_request(r, q, ldq, b, h, q0, N, ssq, groups, g);
  q_finish(r, qf, D, ssq, groups, eps);
}

__global__ __launch_bounds__(64) void cross_attn_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ kc, int ldk,
    const bf16_t* __restrict__ vct, bf16_t* __restrict__ o, int ldo, int N, int La, int D, int hw,
    int apf, int full, float scale_log2, const float* __restrict__ ssq, int groups,
    const float* __restrict__ g, float eps) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = blockIdx.x * 32;

  bf16x8 qf[8];
  load_q_frags(qf, q, ldq, b, h, q0, N, D, ssq, groups, g, eps);
  const int k_lo = full ? 0 : (q0 / hw) * apf;
  const int k_hi = full ? La : k_lo + apf;

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = k_lo; k0 < k_hi; k0 += 32) {
    bf16x8 kf[8], vf[2][4];
    const bf16_t* kp = kc + ((int64_t)b * La + k0 + lr) * ldk + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vf[u][dt] = load_v_frag(vct + ((int64_t)b * D + h * HD + 32 * dt + lr) * La + k0 + 16 * u + 4 * lh);
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], st, 0, 0, 0);
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
      for (int dt = 0; dt < 4; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][dt], pf, acc[dt], 0, 0, 0);
    }
  }
  l_run += __shfl_xor(l_run, 32, 64);
  if (q0 + lr < N) store_o(o + ((int64_t)b * N + q0 + lr) * ldo + h * HD, acc, 1.f / l_run, lh);
}

// Frame-local cross-attention probabilities: for 32 queries of one (lane,
// head), the softmax over the apf audio tokens of their latent frame (at most
// MAXKB blocks of 32, scores kept in registers), written normalised as bf16 to
// p[row][h apf + j]. The value product and the output projection then run as
// one GEMM against per-frame products of the values with that projection.
constexpr int MAXKB = 4;

__global__ __launch_bounds__(64) void cross_probs_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ kc, int ldk, bf16_t* __restrict__ p,
    int ldp, int N, int La, int D, int hw, int apf, float scale_log2, const float* __restrict__ ssq, int groups,
    const float* __restrict__ g, float eps) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  const int q0 = blockIdx.x * 32;

  // the query's loads and the first key block's go out together: one latency
  const int k_lo = (q0 / hw) * apf, nkb = apf / 32;
  bf16x8 qf[8];
  QReq qr;
  q_request(qr, q, ldq, b, h, q0, N, ssq, groups, g);
  bf16x8 kf0[8];
  {
    const bf16_t* kp = kc + ((int64_t)b * La + k_lo + lr) * ldk + h * HD + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf0[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
  }
  q_finish(qr, qf, D, ssq, groups, eps);

  // S^T blocks: lane (lr, lh) holds query lr's scores of keys 8 (r/4) + 4 lh + r%4
  f32x16 st[MAXKB];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < MAXKB; ++kb) {
    if (kb >= nkb) break;
    bf16x8 kf[8];
    if (kb == 0) {
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = kf0[s];
    } else {
      const bf16_t* kp = kc + ((int64_t)b * La + k_lo + 32 * kb + lr) * ldk + h * HD + 8 * lh;
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], st[kb], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r] * scale_log2);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float l = 0.f;
#pragma unroll
  for (int kb = 0; kb < MAXKB; ++kb) {
    if (kb >= nkb) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st[kb][r] = exp2f(fmaf(st[kb][r], scale_log2, -mx));
      l += st[kb][r];
    }
  }
  l += __shfl_xor(l, 32, 64);
  const float inv = 1.f / l;
  if (q0 + lr >= N) return;
  bf16_t* pr = p + ((int64_t)b * N + q0 + lr) * ldp + h * apf + 4 * lh;
#pragma unroll
  for (int kb = 0; kb < MAXKB; ++kb) {
    if (kb >= nkb) break;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x2 w = {pack2bf(st[kb][4 * a] * inv, st[kb][4 * a + 1] * inv),
                       pack2bf(st[kb][4 * a + 2] * inv, st[kb][4 * a + 3] * inv)};
      *reinterpret_cast<u32x2*>(pr + 32 * kb + 8 * a) = w;
    }
  }
}

}  // namespace

hipError_t flash_attn(const bf16_t* q, int ldq, const bf16_t* k, int ldk, const bf16_t* vt,
                      bf16_t* o, int ldo, int B, int N, int n_heads, float scale, hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if (N % 32 || ldq % 8 || ldk % 8 || ldo % 4) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int n_qt = (N + AQ - 1) / AQ, n_wg = n_qt * n_heads * B;
  launch_timed(flash_attn_kernel, dim3((n_wg + 7) / 8 * 8), dim3(256), s, q, ldq, k, ldk, vt, o, ldo, N,
               n_heads * HD, scale_log2, n_qt, n_heads, n_wg);
  return hipGetLastError();
}

hipError_t flash_attn_mx(const uint8_t* q, const uint8_t* qs, const uint8_t* k, const uint8_t* ks, int ldq,
                         const uint8_t* vt, const uint8_t* vts, bf16_t* o, int ldo, int B, int N, int n_heads,
                         float scale, hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if (N % 64 || ldq % 32 || ldq < n_heads * HD || ldo % 4 || !qs || !ks || !vts) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int n_qt = (N + AQ - 1) / AQ, n_wg = n_qt * n_heads * B;
  launch_timed(flash_attn_mx_kernel, dim3((n_wg + 7) / 8 * 8), dim3(256), s, q, qs, k, ks, ldq, vt, vts, o, ldo, N,
               n_heads * HD, scale_log2, n_qt, n_heads, n_wg);
  return hipGetLastError();
}

hipError_t cross_probs(const bf16_t* q, int ldq, const bf16_t* kc, int ldk, bf16_t* p, int ldp, int B, int N,
                       int La, int hw, int apf, int n_heads, float scale, const float* ssq, int groups,
                       const float* g, float eps, hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  // apf >= 32: the kernel reads the first key block of a frame before it knows the count
  if (N % 32 || hw % 32 || apf % 32 || apf < 32 || apf > 32 * MAXKB || La % 32 || ldq % 8 || ldk % 8 || ldp % 4 ||
      ldp < n_heads * apf || (N / hw) * apf > La || !p)
    return hipErrorInvalidValue;
  if (ssq && (groups < 4 || groups > MAXG || groups % 4 || !g)) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(N / 32, n_heads, B);
  launch_timed(cross_probs_kernel, grid, dim3(64), s, q, ldq, kc, ldk, p, ldp, N, La, n_heads * HD, hw, apf,
               scale_log2, ssq, groups, g, eps);
  return hipGetLastError();
}

hipError_t cross_attn(const bf16_t* q, int ldq, const bf16_t* kc, int ldk, const bf16_t* vct,
                      bf16_t* o, int ldo, int B, int N, int La, int hw, int apf, int full,
                      int n_heads, float scale, const float* ssq, int groups, const float* g, float eps,
                      hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if (N % 32 || hw % 32 || apf % 32 || La % 32 || ldq % 8 || ldk % 8 || ldo % 4)
    return hipErrorInvalidValue;
  if (!full && (N / hw) * apf > La) return hipErrorInvalidValue;
  if (ssq && (groups < 4 || groups > MAXG || groups % 4 || !g)) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  dim3 grid(N / 32, n_heads, B);
  launch_timed(cross_attn_kernel, grid, dim3(64), s, q, ldq, kc, ldk, vct, o, ldo, N, La, n_heads * HD, hw, apf,
               full, scale_log2, ssq, groups, g, eps);
  return hipGetLastError();
}

hipError_t set_wg_reverse_attn(int r) { return set_wg_reverse(r); }

}  // namespace fh
