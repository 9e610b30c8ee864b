/*
 * fh.h -- C ABI of libfh, the MI355X (gfx950) slice denoiser of SoulX-FlashHead Lite.
 *
 * What it computes (gizai:flashhead reference page, overview paragraph): a
 * Wan-style transformer -- 30 blocks of width 1536, 12 heads, rotary over
 * frame, row and column -- predicts the flow of one slice's noisy video latent
 * (5 latent frames of 16x16), whose first latent frames are the motion of the
 * previous slice, in 4 steps, conditioned on 5 latent frames of 32 audio
 * tokens. The same page's FlashHead type lists the parameters the library
 * binds: per-block weights, the `patch` and `head` Linear layers, the output
 * norm's per-step shift/scale (`headMods`) and the rotary tables (`cos`,
 * `sin`). The audio-cpp page "SoulX-FlashHead", section "Generate", gives the
 * 4 denoising steps; its section "Variant boundaries" says the transformer
 * dimensions come from a configuration (here fh_config) and that an
 * unavailable implementation is rejected rather than substituted (here:
 * unsupported sizes return FH_EUNSUPPORTED, never a fallback).
 *
 * Conventions for every call:
 *  - All device pointers are caller-owned HIP device memory (inputs, outputs,
 *    weights, workspace). The library never allocates device memory.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Calls
 *    enqueue work on it and return; kernel faults surface at the caller's
 *    next synchronisation.
 *  - A context is not thread-safe: use one per host thread / stream.
 *  - Results are deterministic: the same inputs give the same bits.
 *  - On error a call returns an FH_E* code, enqueues nothing, and
 *    fh_last_error() describes the problem.
 *  - Launch trace: with FH_TRACE=1 in the environment (read once per
 *    process), every kernel launch prints one line to stderr -- kernel name
 *    with its template arguments, grid, block, dynamic LDS bytes, stream and
 *    the kernel's scalar arguments (sizes, strides, scales; pointers as
 *    addresses). Work recorded into a HIP graph prints when the graph is
 *    captured (a call's first run with FH_OPT_GRAPH on), not on replays.
 */
#ifndef FH_H
#define FH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FH_OK = 0,
  FH_EINVAL = 1,        /* null pointer, batch <= 0, n_steps < 0, non-finite sigma, bad block index */
  FH_ESHAPE = 2,        /* a size or weight shape that does not match the configuration */
  FH_EUNSUPPORTED = 3,  /* a configuration the kernels do not implement (e.g. head_dim != 128) */
  FH_EWORKSPACE = 4,    /* workspace pointer null/misaligned or smaller than fh_workspace_bytes() */
  FH_EHIP = 5,          /* a HIP runtime error; its text is kept in fh_last_error() */
  FH_EWEIGHTS = 6       /* a required weight tensor is missing, misaligned or of the wrong dtype */
};

enum { FH_DTYPE_BF16 = 1, FH_DTYPE_F32 = 2, FH_DTYPE_F16 = 3 };

/* Sizes of the DiT and of one slice latent. Every dimension is a runtime value
 * (audio-cpp page, "Variant boundaries"). The kernels implement:
 *   head_dim == 128, dim == n_heads * 128, n_heads even, ffn_dim % 128 == 0,
 *   dim <= 2048, in_ch == out_ch <= 64, freq_dim % 8 == 0, freq_dim <= 2048, frames*height*width
 *   a multiple of 32, height*width a multiple of 32, in_ch a multiple of 16, audio_per_frame a
 *   multiple of 32, 0 <= motion_frames < frames.                                */
typedef struct fh_config {
  int32_t n_blocks;         /* 30 for Lite */
  int32_t dim;              /* model width D, 1536 */
  int32_t n_heads;          /* 12 */
  int32_t head_dim;         /* 128 */
  int32_t ffn_dim;          /* 8960 */
  int32_t in_ch, out_ch;    /* latent channels C, 16 */
  int32_t frames;           /* latent frames F, 5 */
  int32_t height, width;    /* latent rows and columns, 16 x 16 at 512 x 512 */
  int32_t motion_frames;    /* latent frames pinned to the previous slice's motion, 2 */
  int32_t audio_per_frame;  /* audio tokens per latent frame, 32 */
  int32_t freq_dim;         /* sinusoidal timestep embedding width, 256 */
  int32_t cross_full;       /* 0: a token attends to its latent frame's audio tokens; 1: to all */
  float eps;                /* LayerNorm / RMSNorm epsilon, 1e-6 */
  float rope_theta;         /* rotary base, 1e4 */
} fh_config;

/* One entry of a weight index: a tensor inside the caller's device blob. */
typedef struct fh_tensor {
  const char* name;   /* e.g. "blocks.3.qkv.w" (see fh_weight_spec) */
  int32_t dtype;      /* FH_DTYPE_BF16 for DiT matrices, FH_DTYPE_F16 for decoder kernels, FH_DTYPE_F32 for the rest */
  int32_t ndim;       /* 1 or 2 */
  int64_t shape[4];
  uint64_t offset;    /* bytes from the blob start; multiple of 16 */
} fh_tensor;

typedef struct fh_ctx fh_ctx;
typedef struct fh_weights fh_weights;

/* Validate cfg and make a context. Builds no device state and allocates no
 * device memory. Returns FH_EINVAL (null), FH_ESHAPE (inconsistent sizes) or
 * FH_EUNSUPPORTED (sizes the kernels do not implement); *out is NULL then.  */
int fh_create(const fh_config* cfg, fh_ctx** out);

/* Free the context and everything it caches (captured graphs). */
void fh_destroy(fh_ctx* ctx);

/* Number of weight tensors the configuration needs, and the i-th one's name,
 * dtype and shape (offset 0). Matrices are stored [out, in] row-major bf16;
 * biases, gains and modulation tables are f32. Returns FH_EINVAL for a bad i.
 * Names: time_in.{w,b} [D,freq_dim], time_out.{w,b} [D,D], time_proj.{w,b}
 * [6D,D], patch.{w,b} [D,C], head.{w,b} [C,D], head.mod [2,D] (shift, scale),
 * and per block i "blocks.i.": mod [6,D] (shift, scale, gate of the
 * self-attention branch, then of the FFN branch), qkv.{w,b} [3D,D] (rows q,
 * k, v), norm_q.g, norm_k.g [D], o.{w,b} [D,D], norm3.{g,b} [D], cq.{w,b}
 * [D,D], ckv.{w,b} [2D,D] (rows audio k, then v), norm_cq.g, norm_ck.g [D],
 * co.{w,b} [D,D], ffn1.{w,b} [ffn_dim,D], ffn2.{w,b} [D,ffn_dim].            */
int fh_weight_count(const fh_ctx* ctx);
int fh_weight_spec(const fh_ctx* ctx, int i, fh_tensor* out);

/* Bind a caller-owned device blob holding every tensor of fh_weight_spec at
 * the offsets given by `index` (n_index entries, any order). No copy is made:
 * the blob must outlive the returned handle. Every tensor is checked for
 * presence, dtype, shape, 16-byte alignment and bounds (FH_EWEIGHTS).       */
int fh_weights_bind(fh_ctx* ctx, const void* dev_blob, size_t blob_bytes, const fh_tensor* index,
                    int n_index, fh_weights** out);
void fh_weights_release(fh_weights* w);

/* Device workspace (bytes, 256-byte aligned start required) for a batch of
 * `batch` independent lanes: activations, the audio keys/values of every
 * block, the rotary tables and the time embedding (the FlashHead type's
 * `work` scratch), for the context's current precision (FH_PREC_FP32 needs
 * more). With frame-local cross-attention the per-block audio cache also
 * holds the values already multiplied into the cross-attention output
 * projection, per latent frame and head (frames x dim x heads x
 * audio_per_frame bf16 per lane and block: 5.9 MB per block at the Lite
 * sizes). 0 for batch <= 0 or a null ctx.                                    */
size_t fh_workspace_bytes(const fh_ctx* ctx, int batch);

/* One DiT block (block index `block`) on the residual stream, in place.
 *   x      device f32 [batch, N, D], N = frames*height*width, tokens in
 *          (frame, row, column) order; read and overwritten.
 *   temb   device f32 [batch, D]: the time embedding e; the block's
 *          modulation is its table + time_proj(SiLU(e)) split in six rows.
 *   audio  device f32 [batch, frames*audio_per_frame, D], frame-major.
 * Computes: x += gate_sa * O(SelfAttn(RoPE(RMSNorm q/k), LN(x) modulated));
 *           x += CrossO(CrossAttn(LN_affine(x), audio));
 *           x += gate_ff * FFN_gelu_tanh(LN(x) modulated).
 * Errors: FH_EINVAL, FH_EWORKSPACE, FH_EHIP.                                 */
int fh_dit_block_forward(fh_ctx* ctx, const fh_weights* w, int block, int batch, float* x,
                         const float* temb, const float* audio, void* ws, size_t ws_bytes,
                         void* stream);

/* Denoise one slice of each of `batch` lanes with n_steps flow-matching Euler
 * steps (gizai:flashhead page, overview; audio-cpp page "Generate": 4 steps).
 *   latent         device f32 [batch, C, F, H, W]: the noisy latent.
 *   motion_latent  device f32 [batch, C, motion_frames, H, W]: the previous
 *                  slice's motion; written into latent frames [0, motion_frames)
 *                  before the first step and after every step (bitwise).
 *   audio_tokens   device f32 [batch, F*audio_per_frame, D].
 *   sigmas         HOST f32 [n_steps + 1], finite; step i uses timestep
 *                  1000*sigmas[i] and moves the latent by
 *                  (sigmas[i+1] - sigmas[i]) * flow.
 *   latent_out     device f32 [batch, C, F, H, W]; may alias `latent`.
 * n_steps == 0 returns the motion-pinned input. The call enqueues the whole
 * denoise (a captured HIP graph is replayed when graphs are enabled).
 * Errors: FH_EINVAL, FH_EWORKSPACE, FH_EHIP.                                 */
int fh_dit_denoise_slice(fh_ctx* ctx, const fh_weights* w, int batch, const float* latent,
                         const float* motion_latent, const float* audio_tokens, const float* sigmas,
                         int n_steps, float* latent_out, void* ws, size_t ws_bytes, void* stream);

/* Execution options of a context.
 *   FH_OPT_GRAPH: 1 (default) capture fh_dit_denoise_slice into a HIP graph
 *     per (batch, pointers, sigmas, sampler, seed) and replay it; 0 launch
 *     kernels directly.
 *   FH_OPT_TIME_KERNEL: a kernel class (FH_K_*) to time with HIP events on the
 *     call's stream around each of its launches (forces direct launches);
 *     -1 (default) times nothing. fh_kernel_time reads and resets the sums.
 *   FH_OPT_SAMPLER: the update of fh_dit_denoise_slice's steps.
 *     FH_SAMPLER_EULER (default): x' = x + (s' - s) v.
 *     FH_SAMPLER_RENOISE: x' = (1 - s') (x - s v) + s' eps, the re-noising
 *       update the audio-cpp page "SoulX-FlashHead" (section "Variant
 *       boundaries") names for distilled checkpoints, read in the flow-matching
 *       convention x_s = (1 - s) x0 + s eps, v = eps - x0. eps is standard
 *       normal noise drawn per step from the context's seed
 *       (fh_set_noise_seed) by a counter-based generator, so it is
 *       reproducible and independent of launch order: element i (flat index
 *       over [C, F, H, W]) of batch lane b at step k takes Philox-4x32-10
 *       (Salmon et al., SC 2011) at counter (i / 4, b, k, 0) under key (seed
 *       low, high 32 bits); of the four words it uses pair (i mod 4) / 2 as
 *       u = ((w >> 8) + 1) / 2^24 each, and eps = sqrt(-2 ln u_a) times
 *       cos(2 pi u_b) for even i, sin(2 pi u_b) for odd i (Box-Muller).
 *       Motion frames are pinned after every step as with Euler; at s' = 0
 *       the two updates coincide.
 *   FH_OPT_PREFETCH: 1 (default): while the bf16 self-attention output and
 *     cross-attention query projections run, one extra wave per workgroup
 *     reads half each of the block's FFN down-projection weights, and while
 *     the down-projection runs, the next block's attention-output and
 *     cross-query weights, so those GEMMs find them in the memory-side cache
 *     rather than in HBM; 0 turns it off. Results are bit-identical either
 *     way.                                                                 */
enum { FH_OPT_GRAPH = 1, FH_OPT_TIME_KERNEL = 2, FH_OPT_SAMPLER = 3, FH_OPT_PRECISION = 4, FH_OPT_PREFETCH = 5 };
enum { FH_SAMPLER_EULER = 0, FH_SAMPLER_RENOISE = 1 };
/*   FH_OPT_PRECISION: FH_PREC_BF16 (default): bf16 operands everywhere.
 *     FH_PREC_FP8_FFN: the FFN's two GEMMs take MX-FP8 operands on gfx950's
 *       block-scaled MFMA -- the FP8 precision path the page "SoulX-LiveAct,
 *       real-time human animation video from audio and a still image"
 *       credits for the sibling system's speed. Operands are OCP
 *       microscaling FP8: e4m3 elements with one E8M0 power-of-two scale per
 *       32 consecutive elements along K (fh_mxfp8_quantize gives the rule).
 *       The FFN's LayerNorm and GELU emit MX-FP8 directly; the weights need
 *       fh_weights_quantize_fp8 first (FH_EINVAL otherwise). Results differ
 *       from the bf16 path by the FP8 rounding (a few percent).
 *     FH_PREC_FP32: debug precision -- every activation and product in
 *       float32 (bf16 weights widened exactly), plain kernels, for checking
 *       the block structure to ~1e-5. Slow. fh_workspace_bytes grows under
 *       this precision (float32 activations and audio K/V), so query it after
 *       setting the option; a smaller workspace is FH_EWORKSPACE.          */
/*     FH_PREC_FP8_ATTN: FH_PREC_FP8_FFN and the self-attention on MX-FP8
 *       too: the QKV projection on MX-FP8 operands (its LayerNorm writes
 *       codes and scales), q and k quantised along the head dim by the q/k
 *       norm, the values
 *       along the tokens by the QKV projection, the probabilities per query
 *       and 32-key block; both products on the block-scaled MFMA; sums and
 *       softmax in float32. Needs fh_weights_quantize_fp8 and tokens per lane
 *       a multiple of 64 (FH_EUNSUPPORTED otherwise); the workspace grows
 *       (query fh_workspace_bytes after setting it). The gain over
 *       FH_PREC_FP8_FFN comes from the FP8 QKV projection: the attention
 *       kernel itself is softmax-bound and no faster than the bf16 one.    */
/*     FH_PREC_FP8_QKV: FH_PREC_FP8_FFN and the QKV projection on MX-FP8
 *       operands as in FH_PREC_FP8_ATTN (its LayerNorm writes codes and
 *       scales), with q, k and v stored in bf16 and the bf16 self-attention:
 *       the FP8 projection's time without the FP8 attention kernel's. Needs
 *       fh_weights_quantize_fp8; the workspace is FH_PREC_FP8_FFN's.        */
enum { FH_PREC_BF16 = 0, FH_PREC_FP8_FFN = 1, FH_PREC_FP32 = 2, FH_PREC_FP8_ATTN = 3, FH_PREC_FP8_QKV = 4 };
/* Kernel classes of FH_OPT_TIME_KERNEL. FH_K_AUDIO_KV is the once-per-slice
 * audio keys and values of every block (all of its launches as one sample). */
enum {
  FH_K_GEMM_QKV = 0, FH_K_GEMM_O = 1, FH_K_GEMM_CQ = 2, FH_K_GEMM_CO = 3, FH_K_GEMM_FFN1 = 4,
  FH_K_GEMM_FFN2 = 5, FH_K_ATTN = 6, FH_K_CROSS_ATTN = 7, FH_K_LAYERNORM = 8, FH_K_RMSNORM_ROPE = 9,
  FH_K_AUDIO_KV = 10, FH_K_COUNT = 11
};
int fh_set_option(fh_ctx* ctx, int option, int value);
/* Bytes of the device buffer fh_weights_quantize_fp8 fills (0 for a null ctx). */
size_t fh_fp8_weight_bytes(const fh_ctx* ctx);
/* Quantise the FFN and QKV matrices of bound weights to MX-FP8 into a caller-owned
 * device buffer (256-byte aligned, fh_fp8_weight_bytes bytes; it must outlive
 * w) and attach them to w. Enqueued on `stream`. FH_EINVAL for a null,
 * foreign or misaligned argument or a short buffer; FH_EHIP on launch errors. */
int fh_weights_quantize_fp8(fh_ctx* ctx, fh_weights* w, void* dev_buf, size_t bytes, void* stream);
/* The MX-FP8 quantiser used by FH_PREC_FP8_FFN, on caller data: device f32
 * in [rows][K] (K a multiple of 64, 16-byte aligned) -> codes [rows][K] (e4m3
 * bytes) and scales [K/64][rows] uint16 (low byte: E8M0 of the 32-element
 * block 2s, high byte: block 2s + 1). A block with max |x| = a > 0 has
 * shared exponent floor(log2 a) - 8 (>= -127; E8M0 = exponent + 127), an
 * all-zero block 0; codes are x * 2^-exponent clamped to +-448 and rounded
 * to nearest even. FH_EINVAL for bad sizes or pointers, FH_EHIP on errors. */
int fh_mxfp8_quantize(const float* in, int64_t rows, int32_t K, uint8_t* codes, uint16_t* scales, void* stream);

/* The MX-FP8 GEMM of FH_PREC_FP8_FFN on caller data, in the residual form
 * the FFN uses: y[m][n] += sum_k A(m,k) W(n,k) + bias[n] in float32, where
 * A(m,k) and W(n,k) are the decoded values (e4m3 code times 2^(E8M0 - 127)
 * of its 32-element block) of codes a [M][K], w [N][K] with scales
 * a_scales [K/64][M], w_scales [K/64][N] laid out as fh_mxfp8_quantize
 * writes them; y [M][N] and bias [N] are float32 (zero y for a plain
 * product). With part == NULL one pass over K; with part (2*M*N floats of
 * device scratch) K is split in two halves whose sums are added in order
 * (needs M <= 1536, N <= 2048, K >= 4096, K % 128 == 0). Sizes: M even,
 * N % 128 == 0, K % 64 == 0; codes, y, bias and part 16-byte aligned,
 * scales 4-byte aligned. All device pointers, enqueued on `stream`.
 * FH_EINVAL for bad sizes or pointers, FH_EHIP on launch errors.
 * (OCP Microscaling: block-scaled operands of the scaled matrix product.) */
int fh_mxfp8_gemm(const uint8_t* a, const uint16_t* a_scales, const uint8_t* w, const uint16_t* w_scales,
                  int64_t M, int32_t N, int32_t K, const float* bias, float* y, float* part, void* stream);

/* ---- Audio projection front end: speech-encoder states -> the audio tokens
 * fh_dit_denoise_slice takes. The gizai:flashhead page (overview) makes a
 * slice's 5 latent frames of 32 audio tokens from 5 states around each of its
 * 33 frames, out of wav2vec 2.0 base's 12 layers at 200 frames, and names the
 * layers proj1, proj1vf, proj2, proj3 and projNorm (type FlashHead). The
 * arrangement is the plain reading of that:
 *   - states [batch][layers][state_frames][channels], float32; the slice's V =
 *     1 + (frames - 1) * temporal_stride video frames are the last V state frames;
 *   - a frame's feature: the `window` states centred on it (offsets -window/2
 *     .. window - 1 - window/2, clamped to the first and last state), flattened
 *     in (offset, layer, channel) order, width F = window * layers * channels;
 *   - latent frame 0 takes video frame 0's feature, latent frame i >= 1 the
 *     mean of video frames s(i-1)+1 .. s i (s = temporal_stride);
 *   - proj1 (latent frame 0) / proj1vf (the others): F -> hidden, SiLU; proj2:
 *     hidden -> hidden, SiLU; proj3: hidden -> audio_per_frame * dim, the
 *     latent frame's tokens in order; projNorm: LayerNorm over dim with gain
 *     and bias (eps of the configuration);
 *   - tokens [batch][frames * audio_per_frame][dim] float32, latent frame by
 *     latent frame.
 * Matrices bf16 [out, in] (products with float32 accumulation), vectors f32. */
typedef struct fh_audio_config {
  int32_t layers;          /* speech-encoder layers whose states are used (12) */
  int32_t state_frames;    /* state frames over the encoder's window (200: 8 s at 25 per second) */
  int32_t channels;        /* state width (768) */
  int32_t window;          /* states around each video frame (5) */
  int32_t temporal_stride; /* video frames per latent frame after the first (8) */
  int32_t hidden;          /* width of proj1, proj1vf and proj2; a multiple of 128 */
} fh_audio_config;
typedef struct fh_audio_weights fh_audio_weights;

/* Tensors of the front end for `acfg` on this context's DiT sizes: names
 * proj1.{w,b} [hidden, F], proj1vf.{w,b} [hidden, F], proj2.{w,b}
 * [hidden, hidden], proj3.{w,b} [audio_per_frame * dim, hidden], projNorm.{g,b}
 * [dim]. Count 0 (spec FH_EINVAL) for a null or invalid configuration (sizes
 * not positive, F not a multiple of 64, hidden not a multiple of 128).       */
int fh_audio_weight_count(const fh_ctx* ctx, const fh_audio_config* acfg);
int fh_audio_weight_spec(const fh_ctx* ctx, const fh_audio_config* acfg, int i, fh_tensor* out);
/* Bind a caller-owned device blob holding those tensors (checks as
 * fh_weights_bind); the blob must outlive the handle. FH_ESHAPE /
 * FH_EUNSUPPORTED for a bad configuration, FH_EWEIGHTS for a bad index.     */
int fh_audio_weights_bind(fh_ctx* ctx, const fh_audio_config* acfg, const void* dev_blob, size_t blob_bytes,
                          const fh_tensor* index, int n_index, fh_audio_weights** out);
void fh_audio_weights_release(fh_audio_weights* w);
/* Device workspace bytes of fh_audio_project for `batch` lanes (0 for batch <= 0). */
size_t fh_audio_workspace_bytes(const fh_audio_weights* w, int batch);
/* states (device, layout above) -> tokens (device, layout above), enqueued on
 * `stream`. FH_EINVAL for null pointers, foreign weights or batch <= 0,
 * FH_EWORKSPACE for a missing, misaligned (256 bytes) or short workspace.   */
int fh_audio_project(fh_ctx* ctx, const fh_audio_weights* w, int batch, const float* states, float* tokens,
                     void* ws, size_t ws_bytes, void* stream);

/* The slice denoise fed from the speech encoder's states instead of audio
 * tokens, as one call (and, with graphs on, one captured graph): the audio
 * projection front end (fh_audio_project's steps) writes the slice's audio
 * tokens straight into the blocks' bf16 audio buffer, which the per-slice
 * audio K/V of every block then reads (the gizai:flashhead page, overview
 * paragraph and type FlashHead: proj1, proj1vf, proj2, proj3, projNorm feed
 * the blocks' cross-attention). states: device f32 [batch][layers]
 * [state_frames][channels] as fh_audio_project takes them; the other
 * arguments as fh_dit_denoise_slice. The workspace holds the slice's, the
 * front end's and float32 tokens (for FH_PREC_FP32):
 * fh_slice_from_states_workspace_bytes (0 for null or foreign arguments).
 * Errors as fh_dit_denoise_slice, and FH_EINVAL for null or foreign audio
 * weights or states.                                                        */
size_t fh_slice_from_states_workspace_bytes(const fh_ctx* ctx, const fh_audio_weights* aw, int batch);
int fh_dit_denoise_slice_from_states(fh_ctx* ctx, const fh_weights* w, const fh_audio_weights* aw, int batch,
                                     const float* latent, const float* motion_latent, const float* states,
                                     const float* sigmas, int n_steps, float* latent_out, void* ws,
                                     size_t ws_bytes, void* stream);

/* Seed of FH_SAMPLER_RENOISE's noise (default 0). Returns FH_EINVAL for a null ctx. */
int fh_set_noise_seed(fh_ctx* ctx, uint64_t seed);

/* The generator of FH_SAMPLER_RENOISE, exposed for callers that draw matching
 * noise and for testing: out[4 g + j] = word j of Philox-4x32-10 at counter
 * (first_group + g, lane, step, 0) under key (seed low, high 32 bits), for
 * g in [0, n_groups). out is a device buffer of 4 n_groups uint32, 16-byte
 * aligned; the call enqueues one kernel on `stream`. FH_EINVAL for a null or
 * misaligned out, n_groups < 0, or a counter range past 2^32; FH_EHIP if the
 * launch fails.                                                             */
int fh_philox4x32_fill(uint64_t seed, uint32_t lane, uint32_t step, uint32_t first_group, int64_t n_groups,
                       uint32_t* out, void* stream);
/* ---- Colour correction after the decode -----------------------------------
 * The decoded frames' colours matched to the reference picture's (gizai:
 * flashhead reference page, overview paragraph: Lab means and deviations;
 * audio-cpp page "SoulX-FlashHead", section "Generate": the correction
 * strength, 1 by default, 0 disabling it; section "Variant boundaries":
 * colour processing in F32 on the device). Per frame f and Lab channel c,
 * with mu, sd the frame's mean and population deviation and mu_r, sd_r the
 * picture's:  v' = mu_r + (v - mu) sd_r / sd  (mu_r where sd = 0), then
 * v + strength (v' - v), back to sRGB and clamped to [0, 1]. sRGB is
 * IEC 61966-2-1's (BT.709 primaries, its transfer curve, the D65 white at
 * x, y = 0.3127, 0.3290); CIELAB is CIE 15's relative to that white.
 *
 * frames: [3][n_frames][height][width] float32 RGB planes in [0, 1] (a video
 * decoder's channels-first output); picture: [3][ref_height][ref_width]
 * float32 planes, as the reference page's FlashHead.picture makes it; out:
 * like frames, and may be frames itself (in place), but may not overlap it
 * otherwise. Pixel arithmetic is float32, the statistics' sums float64 in a
 * fixed order (deterministic). Device pointers, 4-byte aligned (16-byte
 * aligned with height*width and ref_height*ref_width multiples of 4 takes
 * the vector path), enqueued on `stream`. workspace: caller-owned device
 * memory of fh_color_match_workspace_bytes, 256-byte aligned, unused when
 * strength == 0 (then out is a copy of frames, bit for bit).
 * n_frames == 0 does nothing. FH_EINVAL: sizes out of range (n_frames above
 * 65534, a side <= 0, more than 2^32 - 256 frame pixels in all, either
 * image above 2^32 pixels), a non-finite strength, a null or misaligned pointer,
 * partial overlap; FH_EWORKSPACE: workspace too small; FH_EHIP: launch error.
 * fh_color_match_workspace_bytes returns 0 for sizes fh_color_match rejects
 * or n_frames == 0.                                                          */
size_t fh_color_match_workspace_bytes(int32_t n_frames, int32_t height, int32_t width, int32_t ref_height,
                                      int32_t ref_width);
int fh_color_match(const float* frames, int32_t n_frames, int32_t height, int32_t width, const float* picture,
                   int32_t ref_height, int32_t ref_width, float strength, float* out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* fh_color_match without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The same kernels and results, bit for
 * bit, as fh_color_match; the statistics' partial sums live in a static
 * device array of fh_color_match_noalloc_max_bytes() bytes (4 MiB) that each
 * GPU holds until the process ends. The call allocates nothing. Every call
 * on one GPU shares that array, and a call overwrites every element it reads
 * before reading it, so nothing needs clearing; calls whose work overlaps on
 * one GPU (two streams, or a call and a replay of a graph that captured one)
 * race on it and must be ordered by the caller. Arguments and errors as
 * fh_color_match, except: FH_EWORKSPACE when the call's statistics need more
 * than the array holds (fh_color_match_workspace_bytes of the sizes above
 * fh_color_match_noalloc_max_bytes(): for example 33 frames of 1920 x 1080
 * fit, 33 frames of 3840 x 2160 do not); FH_EHIP if the array's device
 * address cannot be looked up.                                               */
int fh_color_match_noalloc(const float* frames, int32_t n_frames, int32_t height, int32_t width,
                           const float* picture, int32_t ref_height, int32_t ref_width, float strength, float* out,
                           void* stream);
size_t fh_color_match_noalloc_max_bytes(void);

/* ---- Video decoder after the denoiser (an assumed LTX-style layout) --------
 * The gizai:flashhead page (overview paragraph) has the VAE decode the slice
 * latent to 33 frames whose colours are then matched to the picture; the
 * toolkit page gives Lite's LTX stride 32 in space (33 = 1 + 4 x 8 frames from
 * 5 latent frames: stride 8 in time). The layers are not on the pages; this
 * decoder is: conv_in (latent_ch -> widths[0]); three stages of a residual
 * block (x + conv2(SiLU(norm2(conv1(SiLU(norm1(x))))))) and an up-sampling
 * convolution to 8 widths[i+1] channels with depth to space 2 x 2 x 2 that
 * drops the first of the doubled frames (T -> 2T - 1); RMS norm, SiLU,
 * conv_out to out_ch x patch x patch channels unfolded into patch x patch
 * pixels; the result v in [-1, 1] returned as (v + 1) / 2 clamped to [0, 1].
 * Every convolution is 3 x 3 x 3, time padded causally (frame 0 repeated
 * twice before it), space with a zero border; norms are RMS over channels
 * with a gain, eps `eps`. Numerics as the audio-cpp page's "Variant
 * boundaries" section states them for Lite's Conv3D: F16 operands, F32
 * accumulation, F16 output storage with the bias added in F32 to the F16
 * result before the final F16 cast, F16 residual storage, norms accumulated
 * in F32 with F16 output; the latent and the frames are F32.
 * Implemented sizes: latent_ch a power of two in [8, 512]; widths powers of
 * two in [32, 512]; out_ch * patch * patch a multiple of 16 with patch == 4;
 * frames, height, width >= 1, and at most 2^30 output positions per layer.  */
typedef struct fh_vae_config {
  int32_t latent_ch;  /* 16 */
  int32_t frames;     /* latent frames: 5 (-> 33 frames) */
  int32_t height;     /* latent rows: 16 (-> 512) */
  int32_t width;      /* latent columns: 16 (-> 512) */
  int32_t widths[4];  /* decoder channels at the latent resolution and after each up-sampling */
  int32_t out_ch;     /* 3 */
  int32_t patch;      /* 4 */
  float eps;          /* 1e-6 */
} fh_vae_config;
typedef struct fh_vae_weights fh_vae_weights;

/* Tensors of a decoder: count (0 for a configuration outside the implemented
 * sizes) and entry i in blob order. Names: conv_in.{w,b}; up{0,1,2}.norm1.g,
 * .conv1.{w,b}, .norm2.g, .conv2.{w,b}, .up.{w,b}; norm_out.g;
 * conv_out.{w,b}. Kernels are FH_DTYPE_F16 [C_out, 27 C_in] ([C_out][3][3][3]
 * [C_in] row-major: time, row, column taps, then the input channel); biases
 * and gains FH_DTYPE_F32 [C_out]. The up-sampling convolutions' output
 * channel s C' + c (s = 4 dt + 2 dh + dw) fills sub-position (dt, dh, dw) of
 * channel c; conv_out's channel c p^2 + py p + px is pixel (py, px) of
 * colour c. FH_EINVAL for a null argument or i out of range.                 */
int fh_vae_weight_count(const fh_vae_config* cfg);
int fh_vae_weight_spec(const fh_vae_config* cfg, int i, fh_tensor* out);
/* Bind a caller-owned device blob (no copy; it must outlive the binding):
 * every tensor present with its dtype and shape, 16-byte aligned, inside the
 * blob. FH_EINVAL (null arguments or an unsupported configuration),
 * FH_EWEIGHTS (a missing, misplaced or mistyped tensor).                     */
int fh_vae_weights_bind(const fh_vae_config* cfg, const void* blob, size_t blob_bytes, const fh_tensor* index,
                        int n_index, fh_vae_weights** out);
void fh_vae_weights_release(fh_vae_weights* w);
/* Device scratch of one fh_vae_decode call (0 for an unsupported configuration). */
size_t fh_vae_workspace_bytes(const fh_vae_config* cfg);
/* Decode one latent: latent device f32 [latent_ch][frames][height][width];
 * frames device f32 [out_ch][8 (frames - 1) + 1][8 patch height][8 patch width]
 * (RGB planes, the input fh_color_match takes); workspace device memory of
 * fh_vae_workspace_bytes, 256-byte aligned. 16-byte aligned pointers.
 * Enqueued on `stream`. FH_EINVAL (null or misaligned pointers),
 * FH_EWORKSPACE, FH_EHIP (launch errors).                                    */
int fh_vae_decode(const fh_vae_weights* w, const float* latent, float* frames, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Total milliseconds and number of timed launches since the last read.      */
int fh_kernel_time(fh_ctx* ctx, double* total_ms, int64_t* launches);

/* Debugging aid (not a step of the method), process-wide on the current
 * device: reversed = 1 makes every kernel whose waves share LDS (GEMMs,
 * attention, norms, head, decoder convolutions, colour statistics) take its
 * work in the reverse order of workgroup ids, 0 restores the normal order.
 * No reduction depends on scheduling, so results must be bit-identical in
 * both orders; a difference would expose a race through LDS or between
 * workgroups. It waits for the device (a synchronous symbol copy); call it
 * with no library work in flight. FH_EINVAL for other values, FH_EHIP.      */
int fh_debug_workgroup_order(int reversed);

/* Measurement aid (not a step of the method): the shader clock while every
 * compute unit runs back-to-back bf16 MFMAs, in MHz. Launches n_wg
 * workgroups of 256 threads, each timing `iters` MFMA groups with the shader
 * cycle counter against the constant-rate wall clock (hipDeviceAttribute-
 * WallClockRate), on `stream`, and waits for them. dev_buf: caller-owned
 * device buffer of at least 32 * n_wg bytes (4 counters per workgroup).
 * *mhz receives the median over workgroups. FH_EINVAL for null or short
 * arguments, n_wg outside [1, 65536] or iters outside [1, 1 << 20];
 * FH_EHIP on runtime errors.                                                 */
int fh_shader_clock(void* dev_buf, size_t bytes, int n_wg, int iters, void* stream, double* mhz);

/* Human-readable text of the last error on ctx (never NULL), and of a code.  */
const char* fh_last_error(const fh_ctx* ctx);
const char* fh_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FH_H */
