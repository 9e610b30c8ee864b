// Host-side launchers of the libfh HIP kernels (internal to the library).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <string>
#include <type_traits>

#include "fh_common.h"

namespace fh {

// Kernel timing: arm_launch_events(start, stop) makes the next timed launch
// (GEMM, attention) on this thread record start and stop from its own
// dispatch (hipExtLaunchKernel); launch_events_used() then tells (and
// resets) whether a launch took them.
void arm_launch_events(hipEvent_t start, hipEvent_t stop);
bool launch_events_used();
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchEvents& armed_launch_events();  // this thread's

// Launch trace: with FH_TRACE=1 in the environment (read once per process)
// every kernel launch prints one line to stderr: the kernel's name, grid,
// block, dynamic LDS bytes, stream and its scalar arguments (sizes, strides,
// scale factors; pointers as addresses, structures as {}). Launches recorded
// into a HIP graph print when the graph is captured, not when it replays.
bool trace_on();
void trace_line(const void* kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const std::string& args);
template <typename T>
void trace_arg(std::string& out, const T& v) {
  char b[48];
  if constexpr (std::is_same_v<T, bool>) snprintf(b, sizeof b, "%d", (int)v);
  else if constexpr (std::is_integral_v<T> && std::is_signed_v<T>) snprintf(b, sizeof b, "%lld", (long long)v);
  else if constexpr (std::is_integral_v<T>) snprintf(b, sizeof b, "%llu", (unsigned long long)v);
  else if constexpr (std::is_floating_point_v<T>) snprintf(b, sizeof b, "%g", (double)v);
  else if constexpr (std::is_pointer_v<T> || std::is_null_pointer_v<T>) snprintf(b, sizeof b, "%p", (const void*)v);
  else snprintf(b, sizeof b, "{}");
  if (!out.empty()) out += ", ";
  out += b;
}

// a kernel launch that takes the armed events, if any
template <typename Kern, typename... Args>
void launch_timed_lds(Kern kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  if (trace_on()) {
    std::string a;
    (trace_arg(a, args), ...);
    trace_line(reinterpret_cast<const void*>(kern), grid, block, lds, s, a);
  }
  LaunchEvents& e = armed_launch_events();
  if (e.start) {
    hipExtLaunchKernelGGL(kern, grid, block, lds, s, e.start, e.stop, 0, args...);
    e.start = e.stop = nullptr;
    e.used = true;
  } else {
    kern<<<grid, block, lds, s>>>(args...);
  }
}
template <typename Kern, typename... Args>
void launch_timed(Kern kern, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  launch_timed_lds(kern, grid, block, 0, s, args...);
}

// Epilogues of the bf16 GEMM C[M,N] = A[M,K] * W[N,K]^T (+ bias[N]).
enum Epi {
  EPI_BF16 = 0,       // out_bf[m, n] = bf16(C + bias)
  EPI_GELU_BF16 = 1,  // out_bf[m, n] = bf16(gelu_tanh(C + bias))
  EPI_GATED_RES = 2,  // x[m, n] += gate[lane(m), n] * (C + bias)
  EPI_RES = 3,        // x[m, n] += C + bias
  EPI_SPLIT_T = 4,    // n < split: out_bf[m, n] = bf16(C + bias);
                      // n >= split: out_t[lane][n - split][m mod rows] = bf16(C + bias)
  EPI_PARTIAL = 5,    // internal to gemm_bf16 (split K): part[k-part][m, n] = C over that K range
  EPI_BF16_SSQ = 6,   // as EPI_BF16, and ssq[m][p] = sum of the squares of the stored (bf16)
                      // values of row m in column group p (gemm_ssq_groups(M, N, K) groups)
  EPI_GELU_MX = 7,    // gelu_tanh(C + bias) quantised to MX-FP8: out_q[m, n] codes, q_scale
                      // (MX scale layout below, rows = M)
  EPI_SPLIT_T_MX = 8, // n < split as EPI_SPLIT_T; n >= split: C + bias as MX-FP8 along the rows of
                      // each lane (rows a multiple of 64): codes out_q[lane][n - split][m mod rows],
                      // E8M0 scales q_scale_b[lane][(m mod rows) / 64][n - split][block 0 | 1]
};

// MX-FP8 operand layout used by the FP8 GEMM: codes [rows][K] (e4m3 bytes,
// K-contiguous) and the E8M0 scales of the 32-element blocks stored by
// 64-element slab: scale[s][row] = uint16 with block 2s in the low byte and
// block 2s+1 in the high byte (s < K / 64).

// Per-entry pointers of a block-batched launch (the audio K/V of every DiT
// block at once): weights, bias and a norm gain, in device memory.
struct BatchEntry {
  const bf16_t* W;
  const float* bias;
  const float* g;
};
constexpr int MAX_BATCH_TABLE = 64;
struct BatchTableArgs {
  const void* w[MAX_BATCH_TABLE];
  const void* b[MAX_BATCH_TABLE];
  const void* g[MAX_BATCH_TABLE];
  int n;
};
// write n entries of args into dst (device), on the stream (capturable)
hipError_t fill_batch_table(BatchEntry* dst, const BatchTableArgs& args, hipStream_t s);

// Weights a later kernel will read, to be fetched while this kernel runs: up to
// three byte ranges. A prefetching GEMM launch carries one more wave per
// workgroup, which reads its share of the ranges (1 KB pieces, the grid's
// workgroups taking them in turn) into a scratch area of LDS spread over the
// main loop. The data then sits in the memory-side cache when its consumer
// starts, instead of in HBM. Results are unaffected.
struct Prefetch {
  static constexpr int R = 3;
  const void* p[R] = {nullptr, nullptr, nullptr};
  int64_t bytes[R] = {0, 0, 0};
  __host__ __device__ int64_t kb(int i) const { return p[i] ? bytes[i] >> 10 : 0; }  // whole KB pieces of range i
  __host__ __device__ bool any() const { return kb(0) + kb(1) + kb(2) > 0; }
};

struct EpiArgs {
  const float* bias = nullptr;
  bf16_t* out_bf = nullptr;
  int ldo = 0;
  float* x = nullptr;
  int ldx = 0;
  const float* gate_tab = nullptr;  // [N] table row
  const float* gate_e0 = nullptr;   // [lanes, gate_stride] adds (row offset applied by caller)
  int gate_stride = 0;
  int rows_per_lane = 1;            // rows of one batch lane (tokens)
  bf16_t* out_t = nullptr;         // [lanes, t_cols, rows_per_lane]
  int split = 0;
  int t_cols = 0;                   // N - split
  float* part = nullptr;             // EPI_PARTIAL: [splits][M][N]
  size_t part_elems = 0;
  float* ssq = nullptr;              // EPI_BF16_SSQ: [M][groups]
  uint8_t* out_q = nullptr;          // EPI_GELU_MX: codes [M][ldq bytes]
  int ldq = 0;
  uint16_t* q_scale = nullptr;       // EPI_GELU_MX: scales [N / 64][M]
  uint8_t* q_scale_b = nullptr;      // EPI_SPLIT_T_MX: scales of the transposed part
  int ldt = 0;                       // EPI_SPLIT_T: pitch of a transposed row (0: rows_per_lane)
  // row-grouped weights (gemm_bf16_grouped): rows [g R, (g+1) R) of A take W + g * w_group_stride
  int w_group_rows = 0;
  int64_t w_group_stride = 0;
  // block-batched launch (gemm_bf16_batched): entry e of batch takes W, bias from batch[e],
  // A + e batch_a_stride and out_bf / out_t + e batch_out_stride
  const BatchEntry* batch = nullptr;
  int batch_n = 1;
  int64_t batch_a_stride = 0, batch_out_stride = 0;
  Prefetch pf;  // honoured by the 128 x 64 residual and query launches and by split K
};

hipError_t gemm_bf16(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                     const EpiArgs& ep, hipStream_t s);
// Block-diagonal product, one per head: for h < heads, C_h = A[:, h Kh .. +Kh] W[:, h Kh .. +Kh]^T
// (Kh = K / heads), stored transposed: row m = lane l, token t of C_h goes to
// out[(l t_cols + n) ldt + h rows_per_lane + t] (EPI_SPLIT_T with split 0, no bias unless given).
hipError_t gemm_bf16_heads(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, int heads,
                           bf16_t* out, int rows_per_lane, int ldt, hipStream_t s);
// The same product for nb entries of a table in one launch (EPI_BF16, or the head-split
// EPI_SPLIT_T of gemm_bf16_heads with heads > 1): entry e computes
// (A + e a_stride)(W_e)^T (+ bias_e) into out + e out_stride; ep carries the output form.
hipError_t gemm_bf16_batched(int epi, const bf16_t* A, int lda, int64_t a_stride, const BatchEntry* tab, int nb,
                             int ldw, int M, int N, int K, int heads, const EpiArgs& ep, int64_t out_stride,
                             hipStream_t s);
// EPI_RES / EPI_GATED_RES / EPI_BF16 GEMM whose weights change every group_rows rows of A:
// rows [g R, (g+1) R) use W + g * group_stride (R a multiple of 64)
hipError_t gemm_bf16_grouped(int epi, const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                             int group_rows, int64_t group_stride, const EpiArgs& ep, hipStream_t s);
// number of column groups of EPI_BF16_SSQ's per-row partial sums for this shape
int gemm_ssq_groups(int M, int N, int K);

// MX-FP8 GEMM: C = dequant(A) dequant(W)^T on the scaled MFMA, A codes [M][lda
// bytes] with scales As ([K/64][M]), W codes [N][ldw] with scales Ws ([K/64][N]).
// Epilogues as gemm_bf16 (incl. EPI_GELU_MX); K a multiple of 64, N of 128.
hipError_t gemm_mx(int epi, const uint8_t* A, int lda, const uint16_t* As, const uint8_t* W, int ldw,
                   const uint16_t* Ws, int M, int N, int K, const EpiArgs& ep, hipStream_t s);
// split-K form into part[0..1] (as gemm_bf16_splitk)
hipError_t gemm_mx_splitk(const uint8_t* A, int lda, const uint16_t* As, const uint8_t* W, int ldw,
                          const uint16_t* Ws, int M, int N, int K, float* part, size_t part_elems,
                          hipStream_t s);
// quantise rows [rows][K] of f32 (in_f) or bf16 (in_b) values to MX-FP8 codes [rows][K]
// and scales [K/64][rows]; K a multiple of 64
hipError_t mx_quantize(const float* in_f, const bf16_t* in_b, int64_t rows, int K, uint8_t* codes,
                       uint16_t* scales, hipStream_t s);

// A residual update x[m, n] += gate[lane(m), n] * (part[0][m, n] + ... + bias[n])
// that a later kernel applies: a residual GEMM with its K split writes the
// parts, and the next LayerNorm of x (or residual_from_parts) adds them, in
// index order, so the result does not depend on scheduling.
struct PendingRes {
  const float* part = nullptr;       // [nparts][M][N]; nullptr = nothing pending
  int nparts = 0;
  const float* bias = nullptr;       // [N]
  const float* gate_tab = nullptr;   // [N], nullptr = no gate
  const float* gate_e0 = nullptr;    // [lanes, gate_stride]
  int gate_stride = 0;
  int rows_per_lane = 1;
};

// x[m, n..n+3] with the pending update applied (parts are [nparts][M][N]).
__device__ __forceinline__ f32x4 apply_pending(const PendingRes& r, f32x4 x, int m, int n, int M, int N) {
  const int64_t i = (int64_t)m * N + n, MN = (int64_t)M * N;
  f32x4 v = *reinterpret_cast<const f32x4*>(r.part + i);
  for (int k = 1; k < r.nparts; ++k) v = v + *reinterpret_cast<const f32x4*>(r.part + k * MN + i);
  f32x4 u = v + *reinterpret_cast<const f32x4*>(r.bias + n);
  if (r.gate_tab) {
    const f32x4 gt = *reinterpret_cast<const f32x4*>(r.gate_tab + n);
    const f32x4 ge = *reinterpret_cast<const f32x4*>(r.gate_e0 + (int64_t)(m / r.rows_per_lane) * r.gate_stride + n);
    u = u * (gt + ge);
  }
  return x + u;
}

// Split-K form of the residual GEMMs: the two halves of K into part[0..1].
bool gemm_splitk_ok(int M, int N, int K);
// the wider split-K form of gemm_bf16_splitk (192 x 192 tiles, bf16 only) for 1536 < M <= 3072
bool gemm_splitk_wide_ok(int M, int N, int K);
hipError_t gemm_bf16_splitk(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                            float* part, size_t part_elems, hipStream_t s, const Prefetch& pf = Prefetch());
hipError_t residual_from_parts(float* x, int ldx, const PendingRes& r, int M, int N, hipStream_t s);
// Split-K partial products of a small-M GEMM: part[s][m][n] = sum over K range s
// (K / splits columns each) of A[m] . W[n] (64 x 128 tiles; N % 128 == 0,
// K a multiple of 64 * splits, part_elems >= splits * M * N).
hipError_t gemm_bf16_splitk_n(const bf16_t* A, int lda, const bf16_t* W, int ldw, int M, int N, int K, int splits,
                              float* part, size_t part_elems, hipStream_t s);

// Audio projection front end (audio.hip). Window features with the latent
// grouping: X[(i * B + b)][(d * L + l) * C + c], bf16, LF = 1 + (V - 1) / stride.
hipError_t audio_features(const float* states, int B, int L, int T, int C, int W, int V, int stride, int LF,
                          bf16_t* X, hipStream_t s);
// out[row(m)][n] = act(sum_s part[s][m][n] + bias[n]) with row(m) = (m % group) * ngroups
// + m / group (group * ngroups == M); act 0 none, 1 SiLU; float32 out_f or bf16 out_b.
hipError_t sum_parts(const float* part, int splits, int M, int N, const float* bias, int act, int group,
                     int ngroups, float* out_f, bf16_t* out_b, hipStream_t s);

// LayerNorm of fp32 rows (width D) to bf16. Modulated form (g == nullptr):
//   out = LN(x) * (1 + tab_scale + e_scale[lane]) + tab_shift + e_shift[lane]
// Affine form: out = LN(x) * g + b. With a pending residual update (pend and
// pend->part non-null, parts [nparts][rows][D]) x is first updated in place.
// With out_q non-null the output is MX-FP8 instead (codes [rows][D], scales
// [D/64][rows] in q_scale; D a multiple of 64) and out is not written.
hipError_t layernorm_bf16(float* x, bf16_t* out, int rows, int D, int rows_per_lane, float eps,
                          const float* tab_shift, const float* tab_scale, const float* e_shift,
                          const float* e_scale, int e_stride, const float* g, const float* b,
                          const PendingRes* pend, hipStream_t s, uint8_t* out_q = nullptr,
                          uint16_t* q_scale = nullptr);

// In-place RMSNorm over the first D columns of bf16 rows (stride ld), gain g0;
// with nparts == 2 also columns [D, 2D) with gain g1. If cos_t != nullptr the
// normalised values are rotated pairwise: pair j of a head (adjacent dims)
// turns by the angle table [tokens, head_dim/2] row (row mod rows_per_lane).
// With out_q non-null the normalised (and rotated) values are written as
// MX-FP8 instead: codes out_q[row * ldq + part * D + col], E8M0 scales
// q_scale[row * (ldq / 32) + (part * D + col) / 32] (32 columns per block).
hipError_t rmsnorm_rope_bf16(bf16_t* p, int ld, int rows, int D, int nparts, const float* g0,
                             const float* g1, const float* cos_t, const float* sin_t,
                             int rows_per_lane, int head_dim, float eps, hipStream_t s, uint8_t* out_q = nullptr,
                             uint8_t* q_scale = nullptr, int ldq = 0);

// softmax(q k^T * scale) v over all N keys of the same lane; q/k rows of
// stride ldq/ldk (head h at column h*128), values transposed vt[lane][D][N].
hipError_t flash_attn(const bf16_t* q, int ldq, const bf16_t* k, int ldk, const bf16_t* vt,
                      bf16_t* o, int ldo, int B, int N, int n_heads, float scale, hipStream_t s);

// MX-FP8 form of flash_attn: q and k as MX-FP8 along the head dim (codes
// [rows][ldq] bytes, head h at column h*128, scales [rows][ldq/32] bytes), the
// values transposed as MX-FP8 along the keys (codes [lane][D][N], scales
// [lane][N/64][D] byte pairs, as EPI_SPLIT_T_MX writes them); probabilities
// quantised per query and 32-key block; N a multiple of 64.
hipError_t flash_attn_mx(const uint8_t* q, const uint8_t* qs, const uint8_t* k, const uint8_t* ks, int ldq,
                         const uint8_t* vt, const uint8_t* vts, bf16_t* o, int ldo, int B, int N, int n_heads,
                         float scale, hipStream_t s);

// Audio cross-attention with short key ranges: queries of latent frame f =
// row / hw see keys [f*apf, f*apf + apf) (full != 0: all La keys). With ssq
// non-null the queries are first RMS-normalised over their whole row (width
// n_heads*128): row m's sum of squares is ssq[m][0] + ... + ssq[m][groups-1]
// (groups a multiple of 4; added in that order), then q * rsqrt(sum / width +
// eps) * g, rounded to bf16.
hipError_t cross_attn(const bf16_t* q, int ldq, const bf16_t* kc, int ldk, const bf16_t* vct,
                      bf16_t* o, int ldo, int B, int N, int La, int hw, int apf, int full,
                      int n_heads, float scale, const float* ssq, int groups, const float* g, float eps,
                      hipStream_t s);
// Frame-local cross-attention probabilities softmax(q k^T scale) over the apf
// audio tokens of each query's latent frame (apf a multiple of 32, at most 128),
// normalised, bf16, at p[(b N + n) ldp + h apf + j]; query RMSNorm as cross_attn.
hipError_t cross_probs(const bf16_t* q, int ldq, const bf16_t* kc, int ldk, bf16_t* p, int ldp, int B, int N,
                       int La, int hw, int apf, int n_heads, float scale, const float* ssq, int groups,
                       const float* g, float eps, hipStream_t s);

// RMSNorm of rows [rows][D] (pitch ld) in place, row r scaled by tab[r / rows_per_entry].g
hipError_t rmsnorm_bf16_table(bf16_t* p, int ld, int rows, int D, const BatchEntry* tab, int rows_per_entry,
                              float eps, hipStream_t s);

// Rotary angle tables [N, head_dim/2] (cos, sin), computed in float64.
hipError_t rope_table(float* cos_t, float* sin_t, int F, int H, int W, int head_dim, double theta,
                      hipStream_t s);

// Sinusoidal timestep embedding of R timesteps t[r] ([R, dim]).
hipError_t sinusoid(float* out, const float* t_host, int R, int dim, hipStream_t s);

// y[r, n] = act_out(sum_k act_in(x[r, k]) W[n, k] + b[n]); act: 0 none, 1 SiLU.
hipError_t gemv_bf16(const float* x, int R, int K, const bf16_t* W, const float* b, float* y, int N,
                     int act_in, int act_out, hipStream_t s);

// x[lane, n, :] = W_p latent[lane, :, n] + b_p  (latent [B, C, N] fp32).
hipError_t patch_embed(const float* lat, int B, int C, int N, const bf16_t* Wp, const float* bp,
                       float* x, int D, hipStream_t s);

// Output head and Euler update on the modulated, normalised rows h [B*N, D]
// (bf16, from layernorm_bf16 with the head's shift/scale):
//   v = h W_h^T + b_h;  lat_next = token in a motion frame ? motion : lat_cur + dsig * v
// (latents [B, Co, N]; lat_next may alias lat_cur). Co must be a multiple of 16.
// Sampler of the fused head update: Euler, or re-noising with counter-based
// noise of step `step` under the 64-bit seed (k0 low, k1 high word).
struct SamplerArgs {
  int renoise = 0;
  uint32_t step = 0, k0 = 0, k1 = 0;
};
hipError_t head_euler(const bf16_t* h, int B, int N, int D, const bf16_t* Wh, const float* bh, int Co,
                      const float* lat_cur, float* lat_next, const float* motion, int n_motion_tok,
                      float sigma, float sigma_next, const SamplerArgs& sa, hipStream_t s);
// Raw generator words: out[4 g + j] = word j of Philox-4x32-10 at counter
// (first_group + g, lane, step, 0) under key (seed low, high), g < n_groups.
hipError_t philox_fill(uint32_t* out, int64_t n_groups, uint32_t first_group, uint32_t lane, uint32_t step,
                       uint64_t seed, hipStream_t s);

// out = latent with the first n_motion_tok tokens of every (lane, channel) from motion.
hipError_t pin_motion(const float* lat, const float* motion, float* out, int BC, int N,
                      int n_motion_tok, hipStream_t s);

hipError_t f32_to_bf16(const float* in, bf16_t* out, int64_t n, hipStream_t s);
// Video decoder (vae.hip). A causal 3 x 3 x 3 convolution on channels-last F16
// activations in[T][H][W][C_in] (C_in = 2^cin_log2) with kernels w[C_out][27 C_in]
// (tap-major) and F32 bias: F16 sum, + bias in F32, F16 store, then
//   CONV_PLAIN  out[T][H][W][C_out]
//   CONV_RES    out = F16(that + res) (res like out)
//   CONV_UP     depth to space: channel s C' + c (C' = C_out / 8, s = 4 dt + 2 dh + dw) to
//               out[2t + dt - 1][2h + dh][2w + dw][c], frame 2t + dt = 0 dropped
//   CONV_FRAMES channel c 16 + 4 py + px to frames[c][t][4h + py][4w + px] = clamp((v + 1) / 2, 0, 1)
// zero: 16 or more bytes of zeros (the padding row).
// Layers whose tiles cannot fill the chip split K: each split's F32 sums go to
// part ([splits][M][C_out], conv_part_elems elements), and a second kernel
// adds them in index order before the same rounding and store.
enum ConvEpi { CONV_PLAIN = 0, CONV_RES = 1, CONV_UP = 2, CONV_FRAMES = 3, CONV_PART = 4 };
struct ConvArgs {
  const _Float16* in = nullptr;
  int T = 0, H = 0, W = 0, cin_log2 = 0;
  const _Float16* w = nullptr;
  const float* bias = nullptr;
  int cout = 0;
  const _Float16* zero = nullptr;
  _Float16* out = nullptr;
  const _Float16* res = nullptr;
  float* frames = nullptr;
};
hipError_t conv3d_f16(int epi, const ConvArgs& a, float* part, size_t part_elems, hipStream_t s);
size_t conv_part_elems(int T, int H, int W, int cin, int cout);
// RMS norm over the C channels of each of M positions (F32 sums), gain g, SiLU, F16 out
hipError_t norm_silu_f16(const _Float16* x, const float* g, _Float16* y, int64_t M, int C, float eps, hipStream_t s);
// latent [C][F H W] float32 -> channels-last F16; also clears 256 bytes at zero
hipError_t latent_to_f16(const float* lat, int C, int64_t FHW, _Float16* out, _Float16* zero, hipStream_t s);

// the reversed-workgroup-order flag of each source file (fh_common.h, wg_x)
hipError_t set_wg_reverse_gemm(int r);
hipError_t set_wg_reverse_attn(int r);
hipError_t set_wg_reverse_color(int r);
hipError_t set_wg_reverse_norm(int r);
hipError_t set_wg_reverse_misc(int r);
hipError_t set_wg_reverse_vae(int r);

// shader-clock probe: n_wg workgroups of MFMA loops, 4 counters each into out
hipError_t clock_probe(uint64_t* out, int n_wg, int iters, hipStream_t s);

// ---- float32 debug path (FH_PREC_FP32): activations and products in float32 ----
enum EpiF32 {
  F32_OUT = 0,        // out[m, n] = C + bias
  F32_GELU = 1,       // out[m, n] = gelu_tanh(C + bias)
  F32_RES = 2,        // x[m, n] += C + bias
  F32_GATED_RES = 3,  // x[m, n] += (gate_tab[n] + gate_e0[lane(m)][n]) (C + bias)
};
struct EpiF32Args {
  const float* bias = nullptr;
  float* out = nullptr;
  int ldo = 0;
  float* x = nullptr;
  int ldx = 0;
  const float* gate_tab = nullptr;
  const float* gate_e0 = nullptr;
  int gate_stride = 0;
  int rows_per_lane = 1;
};
// C = A W^T with A float32 [M][lda], W bf16 [N][ldw] (N % 64 == 0, K % 16 == 0,
// lda and ldw multiples of 4, A 16-byte and W 8-byte aligned rows).
hipError_t gemm_f32(int epi, const float* A, int lda, const bf16_t* W, int ldw, int M, int N, int K,
                    const EpiF32Args& ep, hipStream_t s);
// LayerNorm of float32 rows to float32, modulated (g == nullptr) or affine, as layernorm_bf16.
hipError_t layernorm_f32(const float* x, float* out, int rows, int D, int rows_per_lane, float eps,
                         const float* tab_shift, const float* tab_scale, const float* e_shift,
                         const float* e_scale, int e_stride, const float* g, const float* b, hipStream_t s);
// In-place RMSNorm (gain g) of the first D columns of float32 rows, then the rotary
// turn of rmsnorm_rope_bf16 when cos_t is non-null.
hipError_t rmsnorm_rope_f32(float* p, int ld, int rows, int D, const float* g, const float* cos_t,
                            const float* sin_t, int rows_per_lane, int head_dim, float eps, hipStream_t s);
// Exact softmax attention in float32, one query row and head per workgroup (head_dim 128):
// lane b's query n sees keys [0, Nk) of lane b, or with local != 0 the apf keys of
// its latent frame n / hw; at most 4096 keys in a range.
hipError_t attn_f32(const float* q, int ldq, const float* k, int ldk, const float* v, int ldv, float* o,
                    int ldo, int B, int Nq, int Nk, int n_heads, float scale, int hw, int apf, int local,
                    hipStream_t s);
// head_euler on float32 rows h [B*N, D].
hipError_t head_euler_f32(const float* h, int B, int N, int D, const bf16_t* Wh, const float* bh, int Co,
                          const float* lat_cur, float* lat_next, const float* motion, int n_motion_tok,
                          float sigma, float sigma_next, const SamplerArgs& sa, hipStream_t s);

// Lab colour match of F frames of npix pixels (planes [3][F][npix]) to a picture
// of npix_ref pixels (planes [3][npix_ref]); out may equal frames. The
// workspace (color_match_workspace bytes, 256-byte aligned) holds the partial
// sums and the per-frame coefficients. Needs 1 <= F <= 65534, npix, npix_ref >= 1.
size_t color_match_workspace(int F, int64_t npix, int64_t npix_ref);
// the static statistics scratch of the allocation-free colour match: its size,
// and the current device's address of it (looked up once per device)
size_t color_scratch_bytes();
hipError_t color_scratch(void** ptr);
hipError_t color_match(const float* frames, int F, int64_t npix, const float* pic, int64_t npix_ref, float strength,
                       float* out, void* ws, hipStream_t s);

}  // namespace fh
