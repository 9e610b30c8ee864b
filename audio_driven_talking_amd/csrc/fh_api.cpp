// libfh host runtime: configuration checks, weight binding, workspace carving,
// the block / slice schedules, HIP graph capture and replay, kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "fh.h"
#include "fh_kernels.h"

namespace {

struct Spec {
  std::string name;
  int dtype;
  int ndim;
  int64_t shape[2];
};

struct WBlock {
  const bf16_t *qkv_w, *o_w, *cq_w, *ckv_w, *co_w, *ffn1_w, *ffn2_w;
  const float *mod, *qkv_b, *norm_q, *norm_k, *o_b, *norm3_g, *norm3_b, *cq_b, *ckv_b, *norm_cq,
      *norm_ck, *co_b, *ffn1_b, *ffn2_b;
  // MX-FP8 copies of the FFN and QKV matrices (fh_weights_quantize_fp8), else null
  const uint8_t *ffn1_q = nullptr, *ffn2_q = nullptr, *qkv_q = nullptr;
  const uint16_t *ffn1_s = nullptr, *ffn2_s = nullptr, *qkv_s = nullptr;
};

struct GraphEntry {
  std::vector<uint64_t> key;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  // recorded on the caller's stream after every launch of exec: an exec may
  // still run when it is evicted or the context is destroyed, so those wait
  // on this event before destroying it
  hipEvent_t done = nullptr;
};

// wait until the last launch of a cached graph has finished, then free it
void release_graph(GraphEntry& ge) {
  if (ge.done) {
    (void)hipEventSynchronize(ge.done);
    (void)hipEventDestroy(ge.done);
  }
  if (ge.exec) (void)hipGraphExecDestroy(ge.exec);
  if (ge.graph) (void)hipGraphDestroy(ge.graph);
  ge = GraphEntry();
}

struct WS {
  float* x;
  bf16_t *h, *qk, *vt, *ao, *qc, *u, *aud, *kc, *vct;
  float *emb, *t1, *e, *e0, *rcos, *rsin;
  float* part;  // split-K partial sums of the width-D residual GEMMs, [2][B*N, D]
  float* ssq;   // per-row column-group sums of squares of the cross-attention queries
  uint8_t *hq, *uq;   // MX-FP8 FFN operands: normalised rows [B*N, D], hidden [B*N, Fd]
  uint16_t *hs, *us;  // and their scales [D/64][B*N], [Fd/64][B*N]
  // float32 activations of FH_PREC_FP32 (carved only for that precision)
  float *fh = nullptr, *fqkv = nullptr, *fao = nullptr, *fqc = nullptr, *fu = nullptr, *fkc = nullptr,
        *fvc = nullptr;
  // MX-FP8 self-attention operands of FH_PREC_FP8_ATTN (carved only for it): q and k codes [B*N][2D]
  // and scales [B*N][2D/32]; V^T codes [B][D][N] and scales [B][N/64][D][2]
  uint8_t *qkq = nullptr, *qks = nullptr, *vq = nullptr, *vs = nullptr;
  // per-block pointer tables of the block-batched audio K/V launches
  fh::BatchEntry *tab_kv = nullptr, *tab_co = nullptr;
  size_t total;
};

constexpr int MAX_GRAPHS = 8;
constexpr int GEMV_ROWS = 8;   // time-MLP rows per GEMV launch (steps of a slice, or lanes)

}  // namespace

struct fh_weights {
  fh_ctx* ctx;
  const bf16_t *time_in_w, *time_out_w, *time_proj_w, *patch_w, *head_w;
  const float *time_in_b, *time_out_b, *time_proj_b, *patch_b, *head_b, *head_mod;
  std::vector<WBlock> blk;
  bool fp8 = false;  // MX-FP8 FFN copies attached
  // identity of this binding's device pointers for the graph cache: new on
  // every bind and every FP8 attach, so a graph captured on other pointers
  // (e.g. of a released binding whose host address is reused) never matches
  uint64_t serial = 0;
};

static std::atomic<uint64_t> g_weights_serial{1};

struct fh_ctx {
  fh_config cfg;
  int N, HW, La;
  // frame-local cross-attention with the value product folded into the output
  // projection (per-frame V' = v W_co^T per head, once per slice)
  bool fold_co = false;
  std::vector<Spec> specs;
  std::string err;
  bool use_graph = true;
  int time_class = -1;
  int sampler = FH_SAMPLER_EULER;
  uint64_t noise_seed = 0;
  int precision = FH_PREC_BF16;
  bool prefetch = true;  // FH_OPT_PREFETCH
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_free, ev_pending;
  double time_ms = 0.0;
  int64_t time_count = 0;
  hipStream_t cap_stream = nullptr;
  std::vector<GraphEntry> graphs;
};

struct fh_audio_weights {
  fh_ctx* ctx;
  fh_audio_config acfg;
  int V, LF, F;  // video frames, latent frames, feature width
  const bf16_t *p1_w, *p1vf_w, *p2_w, *p3_w;
  const float *p1_b, *p1vf_b, *p2_b, *p3_b, *norm_g, *norm_b;
  uint64_t serial = 0;  // identity of this binding for the graph cache
};

namespace {

int fail(fh_ctx* c, int code, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return code;
}

#ifdef FH_DEBUG
// Debug build: every HIP call of the runtime is followed by a device
// synchronisation, so a kernel fault is reported, with the launching call's
// text, by the library call that launched it (graphs are off in this build).
#define FH_HIP(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ == hipSuccess) e_ = hipDeviceSynchronize();                                      \
    if (e_ == hipSuccess) e_ = hipGetLastError();                                           \
    if (e_ != hipSuccess) return fail(c, FH_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)
constexpr bool kDebugBuild = true;
#else
#define FH_HIP(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(c, FH_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)
constexpr bool kDebugBuild = false;
#endif

std::vector<Spec> make_specs(const fh_config& g) {
  const int64_t D = g.dim, Fd = g.ffn_dim, C = g.in_ch, Co = g.out_ch, Fq = g.freq_dim;
  std::vector<Spec> s;
  auto mat = [&](const std::string& n, int64_t a, int64_t b) { s.push_back({n, FH_DTYPE_BF16, 2, {a, b}}); };
  auto vec = [&](const std::string& n, int64_t a) { s.push_back({n, FH_DTYPE_F32, 1, {a, 0}}); };
  auto tab = [&](const std::string& n, int64_t a, int64_t b) { s.push_back({n, FH_DTYPE_F32, 2, {a, b}}); };
  mat("time_in.w", D, Fq); vec("time_in.b", D);
  mat("time_out.w", D, D); vec("time_out.b", D);
  mat("time_proj.w", 6 * D, D); vec("time_proj.b", 6 * D);
  mat("patch.w", D, C); vec("patch.b", D);
  mat("head.w", Co, D); vec("head.b", Co);
  tab("head.mod", 2, D);
  for (int i = 0; i < g.n_blocks; ++i) {
    const std::string p = "blocks." + std::to_string(i) + ".";
    tab(p + "mod", 6, D);
    mat(p + "qkv.w", 3 * D, D); vec(p + "qkv.b", 3 * D);
    vec(p + "norm_q.g", D); vec(p + "norm_k.g", D);
    mat(p + "o.w", D, D); vec(p + "o.b", D);
    vec(p + "norm3.g", D); vec(p + "norm3.b", D);
    mat(p + "cq.w", D, D); vec(p + "cq.b", D);
    mat(p + "ckv.w", 2 * D, D); vec(p + "ckv.b", 2 * D);
    vec(p + "norm_cq.g", D); vec(p + "norm_ck.g", D);
    mat(p + "co.w", D, D); vec(p + "co.b", D);
    mat(p + "ffn1.w", Fd, D); vec(p + "ffn1.b", Fd);
    mat(p + "ffn2.w", D, Fd); vec(p + "ffn2.b", D);
  }
  return s;
}

// per-block audio cache: plain form k [B La][D] and V^T [B][D][La]; folded
// form [k | v] [B La][2D] and V' [B F][D][n_heads apf]
size_t slot_elems(const fh_ctx* c, int B) { return (size_t)B * c->La * c->cfg.dim; }
size_t kslot(const fh_ctx* c, int B) { return (c->fold_co ? 2 : 1) * slot_elems(c, B); }
size_t vslot(const fh_ctx* c, int B) {
  return c->fold_co ? (size_t)B * c->cfg.frames * c->cfg.dim * c->cfg.n_heads * c->cfg.audio_per_frame
                    : slot_elems(c, B);
}

WS carve(const fh_ctx* c, int B, char* base) {
  const fh_config& g = c->cfg;
  const size_t N = c->N, D = g.dim, La = c->La, Fd = g.ffn_dim, nb = g.n_blocks;
  const size_t R = (size_t)(B > GEMV_ROWS ? B : GEMV_ROWS);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  WS w;
  w.x = (float*)take(B * N * D * 4);
  w.h = (bf16_t*)take(B * N * D * 2);
  w.qk = (bf16_t*)take(B * N * 2 * D * 2);
  w.vt = (bf16_t*)take(B * N * D * 2);
  w.ao = (bf16_t*)take(B * N * D * 2);
  w.qc = (bf16_t*)take(B * N * D * 2);
  w.u = (bf16_t*)take(B * N * Fd * 2);
  w.aud = (bf16_t*)take(B * La * D * 2);
  w.kc = (bf16_t*)take(nb * kslot(c, B) * 2);
  w.vct = (bf16_t*)take(nb * vslot(c, B) * 2);
  w.emb = (float*)take(R * g.freq_dim * 4);
  w.t1 = (float*)take(R * D * 4);
  w.e = (float*)take(R * D * 4);
  w.e0 = (float*)take(R * 6 * D * 4);
  w.rcos = (float*)take(N * (g.head_dim / 2) * 4);
  w.rsin = (float*)take(N * (g.head_dim / 2) * 4);
  w.part = (float*)take(2 * B * N * D * 4);
  w.ssq = (float*)take((D / 32) * B * N * 4);
  w.hq = (uint8_t*)take(B * N * D);
  w.hs = (uint16_t*)take((D / 64) * B * N * 2);
  w.uq = (uint8_t*)take(B * N * Fd);
  w.us = (uint16_t*)take((Fd / 64) * B * N * 2);
  w.tab_kv = (fh::BatchEntry*)take(fh::MAX_BATCH_TABLE * sizeof(fh::BatchEntry));
  w.tab_co = (fh::BatchEntry*)take(fh::MAX_BATCH_TABLE * sizeof(fh::BatchEntry));
  if (c->precision == FH_PREC_FP8_ATTN) {
    w.qkq = (uint8_t*)take(B * N * 2 * D);
    w.qks = (uint8_t*)take(B * N * 2 * D / 32);
    w.vq = (uint8_t*)take(B * D * N);
    w.vs = (uint8_t*)take(B * (N / 64) * D * 2);
  }
  if (c->precision == FH_PREC_FP32) {
    w.fh = (float*)take(B * N * D * 4);
    w.fqkv = (float*)take(B * N * 3 * D * 4);
    w.fao = (float*)take(B * N * D * 4);
    w.fqc = (float*)take(B * N * D * 4);
    w.fu = (float*)take(B * N * Fd * 4);
    w.fkc = (float*)take(nb * B * La * D * 4);
    w.fvc = (float*)take(nb * B * La * D * 4);
  }
  w.total = off;
  return w;
}

// -------- kernel timing (events around the launches of one kernel class)
// GEMM classes are one kernel launch each: their events are armed for the
// launch itself (recorded by the dispatch at the kernel's start and end);
// the other classes are bracketed by event records on the stream.
struct Timed {
  fh_ctx* c;
  int cls;
  hipStream_t s;
  bool at_launch = false;
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  Timed(fh_ctx* c_, int cls_, hipStream_t s_) : c(c_), cls(cls_), s(s_) {
    if (c->time_class != cls) return;
    if (!c->ev_free.empty()) {
      ev = c->ev_free.back();
      c->ev_free.pop_back();
    } else {
      if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess) {
        ev = {nullptr, nullptr};
        return;
      }
    }
    at_launch = cls == FH_K_GEMM_QKV || cls == FH_K_GEMM_O || cls == FH_K_GEMM_CQ || cls == FH_K_GEMM_CO ||
                cls == FH_K_GEMM_FFN1 || cls == FH_K_GEMM_FFN2 || cls == FH_K_ATTN || cls == FH_K_CROSS_ATTN;
    if (at_launch) fh::arm_launch_events(ev.first, ev.second);
    else hipEventRecord(ev.first, s);
  }
  ~Timed() {
    if (!ev.first) return;
    if (at_launch) {
      if (!fh::launch_events_used()) {  // no launch took them (an error before it): not a sample
        c->ev_free.push_back(ev);
        return;
      }
    } else {
      hipEventRecord(ev.second, s);
    }
    c->ev_pending.push_back(ev);
  }
};


int audio_kv(fh_ctx* c, const WBlock& wb, int B, bf16_t* kc, bf16_t* vct, const WS& ws, hipStream_t s) {
  const fh_config& g = c->cfg;
  const int D = g.dim;
  if (c->fold_co) {
    // [k | v] row-major, k RMS-normalised in place; then per head h the product
    // v[:, h] W_co[:, h]^T of every latent frame's apf tokens, stored as
    // V'[(lane, frame)][n][h apf + j] for the grouped output projection
    const int apf = g.audio_per_frame, KH = g.n_heads * apf;
    fh::EpiArgs ep;
    ep.bias = wb.ckv_b;
    ep.out_bf = kc;
    ep.ldo = 2 * D;
    FH_HIP(fh::gemm_bf16(fh::EPI_BF16, ws.aud, D, wb.ckv_w, D, B * c->La, 2 * D, D, ep, s));
    FH_HIP(fh::rmsnorm_rope_bf16(kc, 2 * D, B * c->La, D, 1, wb.norm_ck, nullptr, nullptr, nullptr, c->La,
                                 g.head_dim, g.eps, s));
    FH_HIP(fh::gemm_bf16_heads(kc + D, 2 * D, wb.co_w, D, B * c->La, D, D, g.n_heads, vct, apf, KH, s));
    return FH_OK;
  }
  fh::EpiArgs ep;
  ep.bias = wb.ckv_b;
  ep.out_bf = kc;
  ep.ldo = D;
  ep.split = D;
  ep.out_t = vct;
  ep.t_cols = D;
  ep.rows_per_lane = c->La;
  FH_HIP(fh::gemm_bf16(fh::EPI_SPLIT_T, ws.aud, D, wb.ckv_w, D, B * c->La, 2 * D, D, ep, s));
  FH_HIP(fh::rmsnorm_rope_bf16(kc, D, B * c->La, D, 1, wb.norm_ck, nullptr, nullptr, nullptr, c->La,
                               g.head_dim, g.eps, s));
  return FH_OK;
}

// The folded audio K/V of every block in three launches (the per-block form
// of audio_kv, batched over a table of the blocks' weights): [k | v] of all
// blocks, the k RMSNorm of all blocks, V' of all blocks.
int audio_kv_all(fh_ctx* c, const fh_weights* w, int B, const WS& ws, hipStream_t s) {
  const fh_config& g = c->cfg;
  const int D = g.dim, nb = g.n_blocks, apf = g.audio_per_frame, Ma = B * c->La;
  fh::BatchTableArgs kv{}, co{};
  kv.n = co.n = nb;
  for (int i = 0; i < nb; ++i) {
    kv.w[i] = w->blk[i].ckv_w;
    kv.b[i] = w->blk[i].ckv_b;
    kv.g[i] = w->blk[i].norm_ck;
    co.w[i] = w->blk[i].co_w;
  }
  FH_HIP(fh::fill_batch_table(ws.tab_kv, kv, s));
  FH_HIP(fh::fill_batch_table(ws.tab_co, co, s));
  fh::EpiArgs ep;
  ep.out_bf = ws.kc;
  ep.ldo = 2 * D;
  FH_HIP(fh::gemm_bf16_batched(fh::EPI_BF16, ws.aud, D, 0, ws.tab_kv, nb, D, Ma, 2 * D, D, 1, ep, kslot(c, B), s));
  FH_HIP(fh::rmsnorm_bf16_table(ws.kc, 2 * D, nb * Ma, D, ws.tab_kv, Ma, g.eps, s));
  fh::EpiArgs et;
  et.out_t = ws.vct;
  et.split = 0;
  et.t_cols = D;
  et.rows_per_lane = apf;
  et.ldt = g.n_heads * apf;
  FH_HIP(fh::gemm_bf16_batched(fh::EPI_SPLIT_T, ws.kc + D, 2 * D, kslot(c, B), ws.tab_co, nb, D, Ma, D, D,
                               g.n_heads, et, vslot(c, B), s));
  return FH_OK;
}

// pend_in: a residual update left pending by the previous block (applied by
// the first LayerNorm); pend_out: if non-null, the FFN output projection may
// leave its residual update pending there (split K) instead of applying it.
// Half i (0, 1) of a block's FFN down-projection weights as a prefetch range:
// the attention output and cross-attention query GEMMs each read one from HBM
// while they run, so the down-projection finds its weights in the memory-side
// cache (a 30-block slice leaves every block's weights cold).
fh::Prefetch ffn2_half(const WBlock& wb, int D, int Fd, int i) {
  const int64_t total = (int64_t)D * Fd * 2, half = (total / 2) & ~(int64_t)1023;
  fh::Prefetch pf;
  pf.p[0] = reinterpret_cast<const char*>(wb.ffn2_w) + i * half;
  pf.bytes[0] = i ? total - half : half;
  return pf;
}

// The MX-FP8 form (FP8 FFN precisions): the codes (D Fd bytes) in two halves,
// the scales ([Fd / 64][D] u16) with the second.
fh::Prefetch ffn2_half_mx(const WBlock& wb, int D, int Fd, int i) {
  const int64_t total = (int64_t)D * Fd, half = (total / 2) & ~(int64_t)1023;
  fh::Prefetch pf;
  pf.p[0] = reinterpret_cast<const char*>(wb.ffn2_q) + i * half;
  pf.bytes[0] = i ? total - half : half;
  if (i) {
    pf.p[1] = wb.ffn2_s;
    pf.bytes[1] = (int64_t)(Fd / 64) * D * 2;
  }
  return pf;
}

int run_block(fh_ctx* c, const WBlock& wb, int B, float* x, const float* e0, int e0_stride,
              const bf16_t* kc, const bf16_t* vct, const WS& ws, hipStream_t s,
              const fh::PendingRes* pend_in, fh::PendingRes* pend_out, const WBlock* next) {
  const fh_config& g = c->cfg;
  const int N = c->N, D = g.dim, M = B * N, Fd = g.ffn_dim;
  const float scale = 1.0f / std::sqrt((float)g.head_dim);
  // FP8 self-attention: the QKV projection too runs on MX-FP8 operands (the
  // LayerNorm writes codes and scales for it)
  const bool mx_attn = c->precision == FH_PREC_FP8_ATTN;
  const bool mx_qkv = mx_attn || c->precision == FH_PREC_FP8_QKV;  // QKV projection on MX-FP8 operands
  const bool fp8 = c->precision == FH_PREC_FP8_FFN || mx_qkv;
  {
    Timed t(c, FH_K_LAYERNORM, s);
    FH_HIP(fh::layernorm_bf16(x, ws.h, M, D, N, g.eps, wb.mod, wb.mod + D, e0, e0 + D, e0_stride,
                              nullptr, nullptr, pend_in, s, mx_qkv ? ws.hq : nullptr, mx_qkv ? ws.hs : nullptr));
  }
  {
    Timed t(c, FH_K_GEMM_QKV, s);
    fh::EpiArgs ep;
    ep.bias = wb.qkv_b;
    ep.out_bf = ws.qk;
    ep.ldo = 2 * D;
    ep.split = 2 * D;
    ep.out_t = ws.vt;
    ep.t_cols = D;
    ep.rows_per_lane = N;
    if (mx_attn) {  // values straight to MX-FP8 along the tokens
      ep.out_q = ws.vq;
      ep.q_scale_b = ws.vs;
      FH_HIP(fh::gemm_mx(fh::EPI_SPLIT_T_MX, ws.hq, D, ws.hs, wb.qkv_q, D, wb.qkv_s, M, 3 * D, D, ep, s));
    } else if (mx_qkv) {  // bf16 q, k and transposed values for the bf16 attention
      FH_HIP(fh::gemm_mx(fh::EPI_SPLIT_T, ws.hq, D, ws.hs, wb.qkv_q, D, wb.qkv_s, M, 3 * D, D, ep, s));
    } else {
      FH_HIP(fh::gemm_bf16(fh::EPI_SPLIT_T, ws.h, D, wb.qkv_w, D, M, 3 * D, D, ep, s));
    }
  }
  {
    Timed t(c, FH_K_RMSNORM_ROPE, s);
    FH_HIP(fh::rmsnorm_rope_bf16(ws.qk, 2 * D, M, D, 2, wb.norm_q, wb.norm_k, ws.rcos, ws.rsin, N,
                                 g.head_dim, g.eps, s, mx_attn ? ws.qkq : nullptr, mx_attn ? ws.qks : nullptr,
                                 2 * D));
  }
  {
    Timed t(c, FH_K_ATTN, s);
    if (mx_attn)
      FH_HIP(fh::flash_attn_mx(ws.qkq, ws.qks, ws.qkq + D, ws.qks + D / 32, 2 * D, ws.vq, ws.vs, ws.ao, D, B, N,
                               g.n_heads, scale, s));
    else
      FH_HIP(fh::flash_attn(ws.qk, 2 * D, ws.qk + D, 2 * D, ws.vt, ws.ao, D, B, N, g.n_heads, scale, s));
  }
  {
    Timed t(c, FH_K_GEMM_O, s);
    fh::EpiArgs ep;
    ep.bias = wb.o_b;
    ep.x = x;
    ep.ldx = D;
    ep.gate_tab = wb.mod + 2 * D;
    ep.gate_e0 = e0 + 2 * D;
    ep.gate_stride = e0_stride;
    ep.rows_per_lane = N;
    if (c->prefetch) ep.pf = fp8 ? ffn2_half_mx(wb, D, Fd, 0) : ffn2_half(wb, D, Fd, 0);
    FH_HIP(fh::gemm_bf16(fh::EPI_GATED_RES, ws.ao, D, wb.o_w, D, M, D, D, ep, s));
  }
  {
    Timed t(c, FH_K_LAYERNORM, s);
    FH_HIP(fh::layernorm_bf16(x, ws.h, M, D, N, g.eps, nullptr, nullptr, nullptr, nullptr, 0, wb.norm3_g,
                              wb.norm3_b, nullptr, s));
  }
  {
    // the query RMSNorm is split between this GEMM (per-row sums of squares of
    // column groups) and the cross-attention kernel (the scaling)
    Timed t(c, FH_K_GEMM_CQ, s);
    fh::EpiArgs ep;
    ep.bias = wb.cq_b;
    ep.out_bf = ws.qc;
    ep.ldo = D;
    ep.ssq = ws.ssq;
    if (c->prefetch) ep.pf = fp8 ? ffn2_half_mx(wb, D, Fd, 1) : ffn2_half(wb, D, Fd, 1);
    FH_HIP(fh::gemm_bf16(fh::EPI_BF16_SSQ, ws.h, D, wb.cq_w, D, M, D, D, ep, s));
  }
  if (c->fold_co) {
    // probabilities P [M][n_heads apf] (in ao), then x += P V'_frame + b: the value
    // product and the output projection in one GEMM of depth n_heads apf
    const int apf = g.audio_per_frame, KH = g.n_heads * apf;
    {
      Timed t(c, FH_K_CROSS_ATTN, s);
      FH_HIP(fh::cross_probs(ws.qc, D, kc, 2 * D, ws.ao, KH, B, N, c->La, c->HW, apf, g.n_heads, scale, ws.ssq,
                             fh::gemm_ssq_groups(M, D, D), wb.norm_cq, g.eps, s));
    }
    {
      Timed t(c, FH_K_GEMM_CO, s);
      fh::EpiArgs ep;
      ep.bias = wb.co_b;
      ep.x = x;
      ep.ldx = D;
      FH_HIP(fh::gemm_bf16_grouped(fh::EPI_RES, ws.ao, KH, vct, KH, M, D, KH, c->HW, (int64_t)D * KH, ep, s));
    }
  } else {
    {
      Timed t(c, FH_K_CROSS_ATTN, s);
      FH_HIP(fh::cross_attn(ws.qc, D, kc, D, vct, ws.ao, D, B, N, c->La, c->HW, g.audio_per_frame,
                            g.cross_full, g.n_heads, scale, ws.ssq, fh::gemm_ssq_groups(M, D, D),
                            wb.norm_cq, g.eps, s));
    }
    {
      Timed t(c, FH_K_GEMM_CO, s);
      fh::EpiArgs ep;
      ep.bias = wb.co_b;
      ep.x = x;
      ep.ldx = D;
      FH_HIP(fh::gemm_bf16(fh::EPI_RES, ws.ao, D, wb.co_w, D, M, D, D, ep, s));
    }
  }
  {
    Timed t(c, FH_K_LAYERNORM, s);
    FH_HIP(fh::layernorm_bf16(x, ws.h, M, D, N, g.eps, wb.mod + 3 * D, wb.mod + 4 * D, e0 + 3 * D,
                              e0 + 4 * D, e0_stride, nullptr, nullptr, nullptr, s, fp8 ? ws.hq : nullptr,
                              fp8 ? ws.hs : nullptr));
  }
  {
    Timed t(c, FH_K_GEMM_FFN1, s);
    fh::EpiArgs ep;
    ep.bias = wb.ffn1_b;
    if (fp8) {  // MX-FP8 operands, GELU output quantised to MX-FP8 for the next GEMM
      ep.out_q = ws.uq;
      ep.ldq = Fd;
      ep.q_scale = ws.us;
      FH_HIP(fh::gemm_mx(fh::EPI_GELU_MX, ws.hq, D, ws.hs, wb.ffn1_q, D, wb.ffn1_s, M, Fd, D, ep, s));
    } else {
      ep.out_bf = ws.u;
      ep.ldo = Fd;
      FH_HIP(fh::gemm_bf16(fh::EPI_GELU_BF16, ws.h, D, wb.ffn1_w, D, M, Fd, D, ep, s));
    }
  }
  {
    Timed t(c, FH_K_GEMM_FFN2, s);
    fh::EpiArgs ep;
    ep.bias = wb.ffn2_b;
    ep.x = x;
    ep.ldx = D;
    ep.gate_tab = wb.mod + 5 * D;
    ep.gate_e0 = e0 + 5 * D;
    ep.gate_stride = e0_stride;
    ep.rows_per_lane = N;
    if (pend_out && (fh::gemm_splitk_ok(M, D, Fd) || (!fp8 && fh::gemm_splitk_wide_ok(M, D, Fd)))) {
      if (fp8)
        FH_HIP(fh::gemm_mx_splitk(ws.uq, Fd, ws.us, wb.ffn2_q, Fd, wb.ffn2_s, M, D, Fd, ws.part,
                                  (size_t)2 * M * D, s));
      else {
        // the next block's attention output and cross-attention query weights, read from HBM
        // meanwhile
        fh::Prefetch pf;
        if (c->prefetch && next) {
          pf.p[0] = next->o_w;
          pf.p[1] = next->cq_w;
          pf.bytes[0] = pf.bytes[1] = (int64_t)D * D * 2;
        }
        FH_HIP(fh::gemm_bf16_splitk(ws.u, Fd, wb.ffn2_w, Fd, M, D, Fd, ws.part, (size_t)2 * M * D, s, pf));
      }
      pend_out->part = ws.part;
      pend_out->nparts = 2;
      pend_out->bias = ep.bias;
      pend_out->gate_tab = ep.gate_tab;
      pend_out->gate_e0 = ep.gate_e0;
      pend_out->gate_stride = ep.gate_stride;
      pend_out->rows_per_lane = N;
    } else {
      if (pend_out) *pend_out = fh::PendingRes();
      if (fp8)
        FH_HIP(fh::gemm_mx(fh::EPI_GATED_RES, ws.uq, Fd, ws.us, wb.ffn2_q, Fd, wb.ffn2_s, M, D, Fd, ep, s));
      else
        FH_HIP(fh::gemm_bf16(fh::EPI_GATED_RES, ws.u, Fd, wb.ffn2_w, Fd, M, D, Fd, ep, s));
    }
  }
  return FH_OK;
}

// ---- float32 debug precision: the same block in float32 kernels, residual
// updates applied at once (no pending parts)
int audio_kv_f32(fh_ctx* c, const WBlock& wb, int B, const float* audio, float* kc, float* vc, hipStream_t s) {
  const fh_config& g = c->cfg;
  const int D = g.dim, M = B * c->La;
  fh::EpiF32Args ep;
  ep.bias = wb.ckv_b;
  ep.out = kc;
  ep.ldo = D;
  FH_HIP(fh::gemm_f32(fh::F32_OUT, audio, D, wb.ckv_w, D, M, D, D, ep, s));
  ep.bias = wb.ckv_b + D;
  ep.out = vc;
  FH_HIP(fh::gemm_f32(fh::F32_OUT, audio, D, wb.ckv_w + (size_t)D * D, D, M, D, D, ep, s));
  FH_HIP(fh::rmsnorm_rope_f32(kc, D, M, D, wb.norm_ck, nullptr, nullptr, c->La, g.head_dim, g.eps, s));
  return FH_OK;
}

int run_block_f32(fh_ctx* c, const WBlock& wb, int B, float* x, const float* e0, int e0_stride,
                  const float* kc, const float* vc, const WS& ws, hipStream_t s) {
  const fh_config& g = c->cfg;
  const int N = c->N, D = g.dim, M = B * N, Fd = g.ffn_dim;
  const float scale = 1.0f / std::sqrt((float)g.head_dim);
  fh::EpiF32Args gated;
  gated.x = x;
  gated.ldx = D;
  gated.gate_stride = e0_stride;
  gated.rows_per_lane = N;
  // self-attention branch
  FH_HIP(fh::layernorm_f32(x, ws.fh, M, D, N, g.eps, wb.mod, wb.mod + D, e0, e0 + D, e0_stride, nullptr,
                           nullptr, s));
  {
    fh::EpiF32Args ep;
    ep.bias = wb.qkv_b;
    ep.out = ws.fqkv;
    ep.ldo = 3 * D;
    FH_HIP(fh::gemm_f32(fh::F32_OUT, ws.fh, D, wb.qkv_w, D, M, 3 * D, D, ep, s));
  }
  FH_HIP(fh::rmsnorm_rope_f32(ws.fqkv, 3 * D, M, D, wb.norm_q, ws.rcos, ws.rsin, N, g.head_dim, g.eps, s));
  FH_HIP(fh::rmsnorm_rope_f32(ws.fqkv + D, 3 * D, M, D, wb.norm_k, ws.rcos, ws.rsin, N, g.head_dim, g.eps, s));
  FH_HIP(fh::attn_f32(ws.fqkv, 3 * D, ws.fqkv + D, 3 * D, ws.fqkv + 2 * D, 3 * D, ws.fao, D, B, N, N,
                      g.n_heads, scale, c->HW, 0, 0, s));
  gated.bias = wb.o_b;
  gated.gate_tab = wb.mod + 2 * D;
  gated.gate_e0 = e0 + 2 * D;
  FH_HIP(fh::gemm_f32(fh::F32_GATED_RES, ws.fao, D, wb.o_w, D, M, D, D, gated, s));
  // audio cross-attention branch
  FH_HIP(fh::layernorm_f32(x, ws.fh, M, D, N, g.eps, nullptr, nullptr, nullptr, nullptr, 0, wb.norm3_g,
                           wb.norm3_b, s));
  {
    fh::EpiF32Args ep;
    ep.bias = wb.cq_b;
    ep.out = ws.fqc;
    ep.ldo = D;
    FH_HIP(fh::gemm_f32(fh::F32_OUT, ws.fh, D, wb.cq_w, D, M, D, D, ep, s));
  }
  FH_HIP(fh::rmsnorm_rope_f32(ws.fqc, D, M, D, wb.norm_cq, nullptr, nullptr, N, g.head_dim, g.eps, s));
  FH_HIP(fh::attn_f32(ws.fqc, D, kc, D, vc, D, ws.fao, D, B, N, c->La, g.n_heads, scale, c->HW,
                      g.audio_per_frame, g.cross_full ? 0 : 1, s));
  {
    fh::EpiF32Args ep;
    ep.bias = wb.co_b;
    ep.x = x;
    ep.ldx = D;
    FH_HIP(fh::gemm_f32(fh::F32_RES, ws.fao, D, wb.co_w, D, M, D, D, ep, s));
  }
  // FFN branch
  FH_HIP(fh::layernorm_f32(x, ws.fh, M, D, N, g.eps, wb.mod + 3 * D, wb.mod + 4 * D, e0 + 3 * D, e0 + 4 * D,
                           e0_stride, nullptr, nullptr, s));
  {
    fh::EpiF32Args ep;
    ep.bias = wb.ffn1_b;
    ep.out = ws.fu;
    ep.ldo = Fd;
    FH_HIP(fh::gemm_f32(fh::F32_GELU, ws.fh, D, wb.ffn1_w, D, M, Fd, D, ep, s));
  }
  gated.bias = wb.ffn2_b;
  gated.gate_tab = wb.mod + 5 * D;
  gated.gate_e0 = e0 + 5 * D;
  FH_HIP(fh::gemm_f32(fh::F32_GATED_RES, ws.fu, Fd, wb.ffn2_w, Fd, M, D, Fd, gated, s));
  return FH_OK;
}

// ---- audio projection front end
int check_audio_cfg(fh_ctx* c, const fh_audio_config* a) {
  if (!a) return fail(c, FH_EINVAL, "null audio configuration");
  if (a->layers <= 0 || a->state_frames <= 0 || a->channels <= 0 || a->window <= 0 || a->temporal_stride <= 0 ||
      a->hidden <= 0)
    return fail(c, FH_ESHAPE, "audio configuration sizes must be positive");
  const int64_t F = (int64_t)a->window * a->layers * a->channels;
  if (F % 64 || F > (1 << 24) || a->hidden % 128 || a->hidden > 8192)
    return fail(c, FH_EUNSUPPORTED,
                "audio feature width (window x layers x channels) must be a multiple of 64 and hidden of 128");
  return FH_OK;
}

std::vector<Spec> audio_specs(const fh_ctx* c, const fh_audio_config& a) {
  const int64_t F = (int64_t)a.window * a.layers * a.channels, P = a.hidden,
                TD = (int64_t)c->cfg.audio_per_frame * c->cfg.dim, D = c->cfg.dim;
  return {{"proj1.w", FH_DTYPE_BF16, 2, {P, F}},   {"proj1.b", FH_DTYPE_F32, 1, {P, 0}},
          {"proj1vf.w", FH_DTYPE_BF16, 2, {P, F}}, {"proj1vf.b", FH_DTYPE_F32, 1, {P, 0}},
          {"proj2.w", FH_DTYPE_BF16, 2, {P, P}},   {"proj2.b", FH_DTYPE_F32, 1, {P, 0}},
          {"proj3.w", FH_DTYPE_BF16, 2, {TD, P}},  {"proj3.b", FH_DTYPE_F32, 1, {TD, 0}},
          {"projNorm.g", FH_DTYPE_F32, 1, {D, 0}}, {"projNorm.b", FH_DTYPE_F32, 1, {D, 0}}};
}

// splits of a split-K GEMM: the largest divisor of the 64-column slabs that
// keeps the grid within two workgroups per CU
int audio_splits(int M, int N, int K) {
  const int slabs = K / 64, tiles = ((M + 63) / 64) * (N / 128);
  int best = 1;
  for (int d = 1; d <= slabs && d <= 256; ++d)
    if (slabs % d == 0 && (int64_t)d * tiles <= 512) best = d;
  return best;
}

struct AudioWS {
  bf16_t *X, *H1, *H2;
  float *part, *Y;
  size_t total;
};

AudioWS carve_audio(const fh_audio_weights* w, int B, char* base) {
  const fh_config& g = w->ctx->cfg;
  const size_t LF = w->LF, F = w->F, P = w->acfg.hidden, TD = (size_t)g.audio_per_frame * g.dim;
  const size_t M = LF * B;
  size_t parts = (size_t)audio_splits(B, (int)P, (int)F) * B * P;
  if (LF > 1) parts = std::max(parts, (size_t)audio_splits((int)(M - B), (int)P, (int)F) * (M - B) * P);
  parts = std::max(parts, (size_t)audio_splits((int)M, (int)P, (int)P) * M * P);
  parts = std::max(parts, (size_t)audio_splits((int)M, (int)TD, (int)P) * M * TD);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  AudioWS a;
  a.X = (bf16_t*)take(M * F * 2);
  a.H1 = (bf16_t*)take(M * P * 2);
  a.H2 = (bf16_t*)take(M * P * 2);
  a.part = (float*)take(parts * 4);
  a.Y = (float*)take(M * TD * 4);
  a.total = off;
  return a;
}

// The audio projection front end (speech-encoder states -> the slice's audio
// tokens, once per slice): features, four split-K projections, projNorm.
// The tokens go to tokens_f32 ([B][La][D] float32) or, for the DiT's own
// bf16 audio buffer, to tokens_bf16.
int enqueue_front(fh_ctx* c, const fh_audio_weights* w, int B, const float* states, const AudioWS& a,
                  float* tokens_f32, bf16_t* tokens_bf16, hipStream_t s) {
  const fh_config& g = c->cfg;
  const fh_audio_config& ac = w->acfg;
  const int LF = w->LF, F = w->F, P = ac.hidden, TD = g.audio_per_frame * g.dim, M = LF * B;
  FH_HIP(fh::audio_features(states, B, ac.layers, ac.state_frames, ac.channels, ac.window, w->V,
                            ac.temporal_stride, LF, a.X, s));
  auto proj = [&](const bf16_t* A, int lda, const bf16_t* W, const float* bias, int rows, int N, int K, int act,
                  int group, int ngroups, float* out_f, bf16_t* out_b) -> int {
    if (rows <= 0) return FH_OK;
    const int sp = audio_splits(rows, N, K);
    FH_HIP(fh::gemm_bf16_splitk_n(A, lda, W, K, rows, N, K, sp, a.part, (size_t)sp * rows * N, s));
    FH_HIP(fh::sum_parts(a.part, sp, rows, N, bias, act, group, ngroups, out_f, out_b, s));
    return FH_OK;
  };
  int rc = proj(a.X, F, w->p1_w, w->p1_b, B, P, F, 1, B, 1, nullptr, a.H1);            // latent frame 0
  if (!rc) rc = proj(a.X + (size_t)B * F, F, w->p1vf_w, w->p1vf_b, M - B, P, F, 1, M - B, 1, nullptr,
                     a.H1 + (size_t)B * P);                                                 // the others
  if (!rc) rc = proj(a.H1, P, w->p2_w, w->p2_b, M, P, P, 1, M, 1, nullptr, a.H2);
  if (!rc) rc = proj(a.H2, P, w->p3_w, w->p3_b, M, TD, P, 0, B, LF, a.Y, nullptr);         // rows -> lane-major
  if (rc) return rc;
  if (tokens_bf16)  // projNorm straight into bf16 rows (the LayerNorm kernel of the blocks, affine form)
    FH_HIP(fh::layernorm_bf16(a.Y, tokens_bf16, B * c->La, g.dim, c->La, g.eps, nullptr, nullptr, nullptr, nullptr,
                              0, w->norm_g, w->norm_b, nullptr, s));
  else
    FH_HIP(fh::layernorm_f32(a.Y, tokens_f32, B * c->La, g.dim, c->La, g.eps, nullptr, nullptr, nullptr, nullptr, 0,
                             w->norm_g, w->norm_b, s));
  return FH_OK;
}

// A slice fed from speech-encoder states instead of audio tokens.
struct FrontEnd {
  const fh_audio_weights* aw;
  const float* states;
  AudioWS a;
  float* tokens;  // float32 tokens, for the float32 precision
};

// workspace of a slice from states: the slice's own, the front end's, float32 tokens
struct StatesWS {
  char* slice;
  AudioWS front;
  float* tokens;
  size_t total;
};

StatesWS states_ws(const fh_ctx* c, const fh_audio_weights* aw, int B, char* base) {
  StatesWS w;
  const size_t s0 = (carve(c, B, nullptr).total + 255) & ~(size_t)255;
  const size_t s1 = (carve_audio(aw, B, nullptr).total + 255) & ~(size_t)255;
  w.slice = base;
  w.front = carve_audio(aw, B, base ? base + s0 : nullptr);
  w.tokens = base ? (float*)(base + s0 + s1) : nullptr;
  w.total = s0 + s1 + (size_t)B * c->La * c->cfg.dim * 4;
  return w;
}

// The whole slice: audio K/V of every block, motion pin, then per step the
// time embedding, patch embedding, all blocks and the head + Euler update.
int enqueue_slice(fh_ctx* c, const fh_weights* w, int B, const float* latent, const float* motion,
                  const float* audio, const FrontEnd* fe, const float* sigmas, int n_steps, float* out, const WS& ws,
                  hipStream_t s) {
  const fh_config& g = c->cfg;
  const int N = c->N, D = g.dim, C = g.in_ch;
  const int nmt = g.motion_frames * c->HW;
  FH_HIP(fh::pin_motion(latent, motion, out, B * C, N, nmt, s));
  if (n_steps == 0) return FH_OK;
  FH_HIP(fh::rope_table(ws.rcos, ws.rsin, g.frames, g.height, g.width, g.head_dim, g.rope_theta, s));
  const bool f32 = c->precision == FH_PREC_FP32;
  if (fe) {
    // the audio tokens from the speech-encoder states: bf16 straight into the
    // blocks' audio buffer (float32 tokens for the float32 precision)
    int rc = enqueue_front(c, fe->aw, B, fe->states, fe->a, f32 ? fe->tokens : nullptr, f32 ? nullptr : ws.aud, s);
    if (rc) return rc;
    audio = fe->tokens;
  } else if (!f32) {
    FH_HIP(fh::f32_to_bf16(audio, ws.aud, (int64_t)B * c->La * D, s));
  }
  {
    Timed t(c, FH_K_AUDIO_KV, s);
    if (!f32 && c->fold_co && g.n_blocks <= fh::MAX_BATCH_TABLE) {
      int rc = audio_kv_all(c, w, B, ws, s);
      if (rc) return rc;
    } else {
      for (int i = 0; i < g.n_blocks; ++i) {
        int rc = f32 ? audio_kv_f32(c, w->blk[i], B, audio, ws.fkc + i * slot_elems(c, B),
                                    ws.fvc + i * slot_elems(c, B), s)
                     : audio_kv(c, w->blk[i], B, ws.kc + i * kslot(c, B), ws.vct + i * vslot(c, B), ws, s);
        if (rc) return rc;
      }
    }
  }
  for (int c0 = 0; c0 < n_steps; c0 += GEMV_ROWS) {
    // time embedding of up to GEMV_ROWS steps at once (the weights are read once)
    const int R = n_steps - c0 < GEMV_ROWS ? n_steps - c0 : GEMV_ROWS;
    float tv[GEMV_ROWS];
    for (int r = 0; r < R; ++r) tv[r] = 1000.0f * sigmas[c0 + r];
    FH_HIP(fh::sinusoid(ws.emb, tv, R, g.freq_dim, s));
    FH_HIP(fh::gemv_bf16(ws.emb, R, g.freq_dim, w->time_in_w, w->time_in_b, ws.t1, D, 0, 1, s));
    FH_HIP(fh::gemv_bf16(ws.t1, R, D, w->time_out_w, w->time_out_b, ws.e, D, 0, 0, s));
    FH_HIP(fh::gemv_bf16(ws.e, R, D, w->time_proj_w, w->time_proj_b, ws.e0, 6 * D, 1, 0, s));
    for (int st = c0; st < c0 + R; ++st) {
      const float* e = ws.e + (size_t)(st - c0) * D;
      const float* e0 = ws.e0 + (size_t)(st - c0) * 6 * D;
      FH_HIP(fh::patch_embed(out, B, C, N, w->patch_w, w->patch_b, ws.x, D, s));
      fh::SamplerArgs sa;
      sa.renoise = c->sampler == FH_SAMPLER_RENOISE;
      sa.step = (uint32_t)st;
      sa.k0 = (uint32_t)c->noise_seed;
      sa.k1 = (uint32_t)(c->noise_seed >> 32);
      if (f32) {
        for (int i = 0; i < g.n_blocks; ++i) {
          int rc = run_block_f32(c, w->blk[i], B, ws.x, e0, 0, ws.fkc + i * slot_elems(c, B),
                                 ws.fvc + i * slot_elems(c, B), ws, s);
          if (rc) return rc;
        }
        FH_HIP(fh::layernorm_f32(ws.x, ws.fh, B * N, D, N, g.eps, w->head_mod, w->head_mod + D, e, e, 0,
                                 nullptr, nullptr, s));
        FH_HIP(fh::head_euler_f32(ws.fh, B, N, D, w->head_w, w->head_b, g.out_ch, out, out, motion, nmt,
                                  sigmas[st], sigmas[st + 1], sa, s));
        continue;
      }
      // each block's FFN residual update may stay pending until the next LayerNorm
      fh::PendingRes pend;
      for (int i = 0; i < g.n_blocks; ++i) {
        fh::PendingRes next;
        // the block after this one: the next of this step, or the first of the next step
        const WBlock* after = i + 1 < g.n_blocks ? &w->blk[i + 1] : st + 1 < n_steps ? &w->blk[0] : nullptr;
        int rc = run_block(c, w->blk[i], B, ws.x, e0, 0, ws.kc + i * kslot(c, B),
                           ws.vct + i * vslot(c, B), ws, s, &pend, &next, after);
        if (rc) return rc;
        pend = next;
      }
      // head: LN modulated by (head.mod + e), then W_h, Euler step and motion pin
      FH_HIP(fh::layernorm_bf16(ws.x, ws.h, B * N, D, N, g.eps, w->head_mod, w->head_mod + D, e, e, 0,
                                nullptr, nullptr, &pend, s));
      FH_HIP(fh::head_euler(ws.h, B, N, D, w->head_w, w->head_b, g.out_ch, out, out, motion, nmt,
                            sigmas[st], sigmas[st + 1], sa, s));
    }
  }
  return FH_OK;
}

// Device pointers of every tensor of `specs` in a caller's blob, checked for
// presence, dtype, shape, 16-byte alignment and bounds.
int resolve_tensors(fh_ctx* c, const std::vector<Spec>& specs, const void* blob, size_t blob_bytes,
                    const fh_tensor* index, int n_index, std::unordered_map<std::string, const void*>& ptr) {
  if (!blob || !index || n_index <= 0) return fail(c, FH_EINVAL, "null blob or empty index");
  if ((uintptr_t)blob & 15) return fail(c, FH_EWEIGHTS, "blob must be 16-byte aligned");
  std::unordered_map<std::string, const fh_tensor*> by_name;
  for (int i = 0; i < n_index; ++i) {
    if (!index[i].name) return fail(c, FH_EINVAL, "index entry %d has no name", i);
    by_name[index[i].name] = &index[i];
  }
  for (const Spec& s : specs) {
    auto it = by_name.find(s.name);
    if (it == by_name.end()) return fail(c, FH_EWEIGHTS, "weight '%s' missing from the index", s.name.c_str());
    const fh_tensor& t = *it->second;
    if (t.dtype != s.dtype)
      return fail(c, FH_EWEIGHTS, "weight '%s' has dtype %d, expected %d", s.name.c_str(), t.dtype, s.dtype);
    if (t.ndim != s.ndim || t.shape[0] != s.shape[0] || (s.ndim == 2 && t.shape[1] != s.shape[1]))
      return fail(c, FH_EWEIGHTS, "weight '%s' has the wrong shape", s.name.c_str());
    const size_t elems = (size_t)s.shape[0] * (s.ndim == 2 ? (size_t)s.shape[1] : 1);
    const size_t bytes = elems * (s.dtype == FH_DTYPE_F32 ? 4 : 2);
    if (t.offset % 16) return fail(c, FH_EWEIGHTS, "weight '%s' offset is not 16-byte aligned", s.name.c_str());
    if (t.offset > blob_bytes || bytes > blob_bytes - t.offset)
      return fail(c, FH_EWEIGHTS, "weight '%s' lies outside the blob", s.name.c_str());
    ptr[s.name] = (const char*)blob + t.offset;
  }
  return FH_OK;
}

int check_precision(fh_ctx* c, const fh_weights* w) {
  if (c->precision == FH_PREC_FP8_ATTN && c->N % 64)
    return fail(c, FH_EUNSUPPORTED, "FP8 self-attention needs tokens per lane a multiple of 64 (have %d)", c->N);
  const bool fp8 = c->precision == FH_PREC_FP8_FFN || c->precision == FH_PREC_FP8_ATTN ||
                   c->precision == FH_PREC_FP8_QKV;
  if (fp8 && !w->fp8)
    return fail(c, FH_EINVAL, "FP8 precision needs fh_weights_quantize_fp8 on these weights");
  return FH_OK;
}

bool check_ws(fh_ctx* c, int B, void* ws, size_t ws_bytes, int* rc) {
  const size_t need = carve(c, B, nullptr).total;
  if (!ws || ((uintptr_t)ws & 255)) {
    *rc = fail(c, FH_EWORKSPACE, "workspace must be a non-null 256-byte aligned device pointer");
    return false;
  }
  if (ws_bytes < need) {
    *rc = fail(c, FH_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes batch %d needs",
               ws_bytes, need, B);
    return false;
  }
  return true;
}

// ---- video decoder
bool vae_cfg_ok(const fh_vae_config* v) {
  auto pow2 = [](int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; };
  if (!v || !pow2(v->latent_ch, 8, 512) || v->frames < 1 || v->height < 1 || v->width < 1 || v->patch != 4 ||
      v->out_ch < 1 || (v->out_ch * v->patch * v->patch) % 16 || !(v->eps > 0.f) || !std::isfinite(v->eps))
    return false;
  for (int i = 0; i < 4; ++i)
    if (!pow2(v->widths[i], 32, 512)) return false;
  // every layer's output positions (the largest is the last resolution) within 2^30
  const int64_t T = 8 * (int64_t)(v->frames - 1) + 1, H = 8 * (int64_t)v->height, W = 8 * (int64_t)v->width;
  return T * H * W <= ((int64_t)1 << 30) && v->frames <= 4096 && v->height <= 4096 && v->width <= 4096;
}

std::vector<Spec> vae_specs(const fh_vae_config& v) {
  std::vector<Spec> s;
  auto conv = [&](const std::string& n, int64_t co, int64_t ci) {
    s.push_back({n + ".w", FH_DTYPE_F16, 2, {co, 27 * ci}});
    s.push_back({n + ".b", FH_DTYPE_F32, 1, {co, 0}});
  };
  auto vec = [&](const std::string& n, int64_t a) { s.push_back({n, FH_DTYPE_F32, 1, {a, 0}}); };
  conv("conv_in", v.widths[0], v.latent_ch);
  for (int i = 0; i < 3; ++i) {
    const std::string p = "up" + std::to_string(i) + ".";
    vec(p + "norm1.g", v.widths[i]);
    conv(p + "conv1", v.widths[i], v.widths[i]);
    vec(p + "norm2.g", v.widths[i]);
    conv(p + "conv2", v.widths[i], v.widths[i]);
    conv(p + "up", 8 * v.widths[i + 1], v.widths[i]);
  }
  vec("norm_out.g", v.widths[3]);
  conv("conv_out", v.out_ch * v.patch * v.patch, v.widths[3]);
  return s;
}

struct VaeWS {
  _Float16 *zero, *x0, *a, *b, *c;
  float* part;  // split-K partial sums of the layers that need them
  size_t part_elems, total;
};

VaeWS carve_vae(const fh_vae_config& v, char* base) {
  int64_t T = v.frames, H = v.height, W = v.width, act = T * H * W * v.widths[0];
  size_t parts = fh::conv_part_elems((int)T, (int)H, (int)W, v.latent_ch, v.widths[0]);
  for (int i = 0; i < 3; ++i) {
    act = std::max(act, T * H * W * v.widths[i]);
    parts = std::max(parts, fh::conv_part_elems((int)T, (int)H, (int)W, v.widths[i], v.widths[i]));
    parts = std::max(parts, fh::conv_part_elems((int)T, (int)H, (int)W, v.widths[i], 8 * v.widths[i + 1]));
    T = 2 * T - 1;
    H *= 2;
    W *= 2;
    act = std::max(act, T * H * W * v.widths[i + 1]);
  }
  parts = std::max(parts, fh::conv_part_elems((int)T, (int)H, (int)W, v.widths[3], v.out_ch * v.patch * v.patch));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return (_Float16*)p;
  };
  VaeWS w;
  w.zero = take(256);
  w.x0 = take((size_t)v.latent_ch * v.frames * v.height * v.width * 2);
  w.a = take((size_t)act * 2);
  w.b = take((size_t)act * 2);
  w.c = take((size_t)act * 2);
  w.part = (float*)take(parts * 4);
  w.part_elems = parts;
  w.total = off;
  return w;
}

int log2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace

struct fh_vae_weights {
  fh_vae_config cfg;
  std::unordered_map<std::string, const void*> ptr;
};

namespace {
int denoise_slice(fh_ctx* c, const fh_weights* w, int batch, const float* latent, const float* motion_latent,
                  const float* audio_tokens, const FrontEnd* fe, const float* sigmas, int n_steps, float* latent_out,
                  void* ws, size_t ws_bytes, void* stream);
}  // namespace

extern "C" {

int fh_create(const fh_config* cfg, fh_ctx** out) {
  if (!out) return FH_EINVAL;
  *out = nullptr;
  if (!cfg) return FH_EINVAL;
  const fh_config& g = *cfg;
  if (g.n_blocks <= 0 || g.dim <= 0 || g.n_heads <= 0 || g.head_dim <= 0 || g.ffn_dim <= 0 ||
      g.in_ch <= 0 || g.out_ch <= 0 || g.frames <= 0 || g.height <= 0 || g.width <= 0 ||
      g.motion_frames < 0 || g.audio_per_frame <= 0 || g.freq_dim <= 0 ||
      (g.cross_full != 0 && g.cross_full != 1) || !(g.eps > 0.f) || !std::isfinite(g.eps) ||
      !(g.rope_theta > 1.f) || !std::isfinite(g.rope_theta))
    return FH_ESHAPE;
  if (g.dim != g.n_heads * g.head_dim || g.in_ch != g.out_ch || g.motion_frames >= g.frames)
    return FH_ESHAPE;
  // n_heads even: the cross-attention query's sums of squares come in column
  // groups of 64 for some tile shapes (dim / 64 of them), which the kernels
  // take four at a time. freq_dim <= 2048: the time-embedding GEMV holds up to
  // 8 rows of its input in 64 KiB of LDS.
  if (g.head_dim != 128 || g.dim % 128 || g.ffn_dim % 128 || g.dim > 2048 || g.in_ch > 64 ||
      g.in_ch % 16 || g.n_heads % 2 ||
      g.freq_dim % 8 || g.freq_dim > 2048 || (g.height * g.width) % 32 || g.audio_per_frame % 32)
    return FH_EUNSUPPORTED;
  fh_ctx* ctx = new fh_ctx();
  ctx->cfg = g;
  ctx->HW = g.height * g.width;
  ctx->N = g.frames * ctx->HW;
  ctx->La = g.frames * g.audio_per_frame;
  ctx->fold_co = !g.cross_full && ctx->HW % 64 == 0 && g.audio_per_frame <= 128 &&
                 (g.n_heads * g.audio_per_frame) % 64 == 0;
  ctx->specs = make_specs(g);
  ctx->use_graph = !kDebugBuild;  // the debug build synchronises after every launch: no capture
  *out = ctx;
  return FH_OK;
}

void fh_destroy(fh_ctx* c) {
  if (!c) return;
  for (auto& ge : c->graphs) release_graph(ge);
  for (auto& e : c->ev_free) { hipEventDestroy(e.first); hipEventDestroy(e.second); }
  for (auto& e : c->ev_pending) { hipEventDestroy(e.first); hipEventDestroy(e.second); }
  if (c->cap_stream) hipStreamDestroy(c->cap_stream);
  delete c;
}

int fh_weight_count(const fh_ctx* c) { return c ? (int)c->specs.size() : 0; }

int fh_weight_spec(const fh_ctx* c, int i, fh_tensor* out) {
  if (!c || !out || i < 0 || i >= (int)c->specs.size()) return FH_EINVAL;
  const Spec& s = c->specs[i];
  std::memset(out, 0, sizeof *out);
  out->name = s.name.c_str();
  out->dtype = s.dtype;
  out->ndim = s.ndim;
  out->shape[0] = s.shape[0];
  out->shape[1] = s.shape[1];
  return FH_OK;
}

int fh_weights_bind(fh_ctx* c, const void* blob, size_t blob_bytes, const fh_tensor* index, int n_index,
                    fh_weights** out) {
  if (!c) return FH_EINVAL;
  if (!out) return fail(c, FH_EINVAL, "out is NULL");
  *out = nullptr;
  std::unordered_map<std::string, const void*> ptr;
  const int rc = resolve_tensors(c, c->specs, blob, blob_bytes, index, n_index, ptr);
  if (rc) return rc;
  fh_weights* w = new fh_weights();
  w->serial = g_weights_serial++;
  w->ctx = c;
  auto M = [&](const std::string& n) { return (const bf16_t*)ptr[n]; };
  auto V = [&](const std::string& n) { return (const float*)ptr[n]; };
  w->time_in_w = M("time_in.w"); w->time_in_b = V("time_in.b");
  w->time_out_w = M("time_out.w"); w->time_out_b = V("time_out.b");
  w->time_proj_w = M("time_proj.w"); w->time_proj_b = V("time_proj.b");
  w->patch_w = M("patch.w"); w->patch_b = V("patch.b");
  w->head_w = M("head.w"); w->head_b = V("head.b"); w->head_mod = V("head.mod");
  for (int i = 0; i < c->cfg.n_blocks; ++i) {
    const std::string p = "blocks." + std::to_string(i) + ".";
    WBlock b;
    b.mod = V(p + "mod");
    b.qkv_w = M(p + "qkv.w"); b.qkv_b = V(p + "qkv.b");
    b.norm_q = V(p + "norm_q.g"); b.norm_k = V(p + "norm_k.g");
    b.o_w = M(p + "o.w"); b.o_b = V(p + "o.b");
    b.norm3_g = V(p + "norm3.g"); b.norm3_b = V(p + "norm3.b");
    b.cq_w = M(p + "cq.w"); b.cq_b = V(p + "cq.b");
    b.ckv_w = M(p + "ckv.w"); b.ckv_b = V(p + "ckv.b");
    b.norm_cq = V(p + "norm_cq.g"); b.norm_ck = V(p + "norm_ck.g");
    b.co_w = M(p + "co.w"); b.co_b = V(p + "co.b");
    b.ffn1_w = M(p + "ffn1.w"); b.ffn1_b = V(p + "ffn1.b");
    b.ffn2_w = M(p + "ffn2.w"); b.ffn2_b = V(p + "ffn2.b");
    w->blk.push_back(b);
  }
  *out = w;
  return FH_OK;
}

void fh_weights_release(fh_weights* w) { delete w; }

size_t fh_workspace_bytes(const fh_ctx* c, int batch) {
  if (!c || batch <= 0) return 0;
  return carve(c, batch, nullptr).total;
}

int fh_dit_block_forward(fh_ctx* c, const fh_weights* w, int block, int batch, float* x, const float* temb,
                         const float* audio, void* ws, size_t ws_bytes, void* stream) {
  if (!c) return FH_EINVAL;
  if (!w || w->ctx != c) return fail(c, FH_EINVAL, "weights are null or bound to another context");
  if (batch <= 0) return fail(c, FH_EINVAL, "batch must be positive, got %d", batch);
  if (block < 0 || block >= c->cfg.n_blocks)
    return fail(c, FH_EINVAL, "block %d outside [0, %d)", block, c->cfg.n_blocks);
  if (!x || !temb || !audio) return fail(c, FH_EINVAL, "null x, temb or audio");
  int rc = FH_OK;
  if (!check_ws(c, batch, ws, ws_bytes, &rc)) return rc;
  rc = check_precision(c, w);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const fh_config& g = c->cfg;
  const int D = g.dim;
  WS wsp = carve(c, batch, (char*)ws);
  FH_HIP(fh::rope_table(wsp.rcos, wsp.rsin, g.frames, g.height, g.width, g.head_dim, g.rope_theta, s));
  const bool f32 = c->precision == FH_PREC_FP32;
  if (f32) {
    rc = audio_kv_f32(c, w->blk[block], batch, audio, wsp.fkc, wsp.fvc, s);
  } else {
    FH_HIP(fh::f32_to_bf16(audio, wsp.aud, (int64_t)batch * c->La * D, s));
    rc = audio_kv(c, w->blk[block], batch, wsp.kc, wsp.vct, wsp, s);
  }
  if (rc) return rc;
  for (int r0 = 0; r0 < batch; r0 += GEMV_ROWS) {
    const int R = batch - r0 < GEMV_ROWS ? batch - r0 : GEMV_ROWS;
    FH_HIP(fh::gemv_bf16(temb + (size_t)r0 * D, R, D, w->time_proj_w, w->time_proj_b,
                         wsp.e0 + (size_t)r0 * 6 * D, 6 * D, 1, 0, s));
  }
  if (f32) return run_block_f32(c, w->blk[block], batch, x, wsp.e0, 6 * D, wsp.fkc, wsp.fvc, wsp, s);
  // the same arithmetic as inside a slice: a pending FFN residual is applied at the end
  fh::PendingRes pend;
  rc = run_block(c, w->blk[block], batch, x, wsp.e0, 6 * D, wsp.kc, wsp.vct, wsp, s, nullptr, &pend, nullptr);
  if (rc) return rc;
  FH_HIP(fh::residual_from_parts(x, D, pend, batch * c->N, D, s));
  return FH_OK;
}

int fh_dit_denoise_slice(fh_ctx* c, const fh_weights* w, int batch, const float* latent,
                         const float* motion_latent, const float* audio_tokens, const float* sigmas,
                         int n_steps, float* latent_out, void* ws, size_t ws_bytes, void* stream) {
  if (!c) return FH_EINVAL;
  if (!audio_tokens) return fail(c, FH_EINVAL, "null audio tokens");
  return denoise_slice(c, w, batch, latent, motion_latent, audio_tokens, nullptr, sigmas, n_steps, latent_out, ws,
                       ws_bytes, stream);
}

}  // extern "C"

namespace {
int denoise_slice(fh_ctx* c, const fh_weights* w, int batch, const float* latent, const float* motion_latent,
                  const float* audio_tokens, const FrontEnd* fe, const float* sigmas, int n_steps, float* latent_out,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!w || w->ctx != c) return fail(c, FH_EINVAL, "weights are null or bound to another context");
  if (batch <= 0) return fail(c, FH_EINVAL, "batch must be positive, got %d", batch);
  if (n_steps < 0) return fail(c, FH_EINVAL, "n_steps must be >= 0, got %d", n_steps);
  if (!latent || !latent_out || (!motion_latent && c->cfg.motion_frames > 0) || (!audio_tokens && !fe) ||
      (!sigmas && n_steps > 0))
    return fail(c, FH_EINVAL, "null latent, motion, audio, sigmas or output pointer");
  for (int i = 0; i <= n_steps && n_steps > 0; ++i)
    if (!std::isfinite(sigmas[i])) return fail(c, FH_EINVAL, "sigma[%d] is not finite", i);
  int rc = FH_OK;
  if (!check_ws(c, batch, ws, ws_bytes, &rc)) return rc;
  rc = check_precision(c, w);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  WS wsp = carve(c, batch, (char*)ws);

  if (!c->use_graph || c->time_class >= 0)
    return enqueue_slice(c, w, batch, latent, motion_latent, audio_tokens, fe, sigmas, n_steps, latent_out, wsp, s);

  std::vector<uint64_t> key = {w->serial, (uint64_t)batch, (uint64_t)(uintptr_t)latent,
                               (uint64_t)(uintptr_t)motion_latent, (uint64_t)(uintptr_t)audio_tokens,
                               fe ? fe->aw->serial : 0, fe ? (uint64_t)(uintptr_t)fe->states : 0,
                               fe ? (uint64_t)(uintptr_t)fe->tokens : 0,
                               (uint64_t)(uintptr_t)latent_out, (uint64_t)(uintptr_t)ws,
                               (uint64_t)n_steps, (uint64_t)c->sampler, c->noise_seed,
                               (uint64_t)c->precision, (uint64_t)c->prefetch};
  for (int i = 0; i <= n_steps && n_steps > 0; ++i) {
    uint32_t b;
    std::memcpy(&b, &sigmas[i], 4);
    key.push_back(b);
  }
  for (auto& ge : c->graphs)
    if (ge.key == key) {
      FH_HIP(hipGraphLaunch(ge.exec, s));
      FH_HIP(hipEventRecord(ge.done, s));
      return FH_OK;
    }
  if (!c->cap_stream) FH_HIP(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  FH_HIP(hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
  rc = enqueue_slice(c, w, batch, latent, motion_latent, audio_tokens, fe, sigmas, n_steps, latent_out, wsp,
                     c->cap_stream);
  hipGraph_t graph = nullptr;
  hipError_t ce = hipStreamEndCapture(c->cap_stream, &graph);
  if (rc != FH_OK) {
    if (graph) hipGraphDestroy(graph);
    return rc;
  }
  if (ce != hipSuccess) return fail(c, FH_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(ce));
  GraphEntry ge;
  ge.key = key;
  ge.graph = graph;
  hipError_t ie = hipGraphInstantiate(&ge.exec, graph, nullptr, nullptr, 0);
  if (ie == hipSuccess) ie = hipEventCreateWithFlags(&ge.done, hipEventDisableTiming);
  if (ie != hipSuccess) {
    release_graph(ge);
    return fail(c, FH_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(ie));
  }
  if ((int)c->graphs.size() >= MAX_GRAPHS) {
    // the oldest graph may still be running from an earlier call: its event
    // waits for that launch before the exec is destroyed
    release_graph(c->graphs.front());
    c->graphs.erase(c->graphs.begin());
  }
  c->graphs.push_back(ge);
  FH_HIP(hipGraphLaunch(ge.exec, s));
  FH_HIP(hipEventRecord(ge.done, s));
  return FH_OK;
}
}  // namespace

extern "C" {

int fh_set_option(fh_ctx* c, int option, int value) {
  if (!c) return FH_EINVAL;
  if (option == FH_OPT_GRAPH) {
    c->use_graph = value != 0 && !kDebugBuild;
    return FH_OK;
  }
  if (option == FH_OPT_TIME_KERNEL) {
    if (value < -1 || value >= FH_K_COUNT) return fail(c, FH_EINVAL, "unknown kernel class %d", value);
    c->time_class = value;
    return FH_OK;
  }
  if (option == FH_OPT_PRECISION) {
    if (value != FH_PREC_BF16 && value != FH_PREC_FP8_FFN && value != FH_PREC_FP32 && value != FH_PREC_FP8_ATTN &&
        value != FH_PREC_FP8_QKV)
      return fail(c, FH_EINVAL, "unknown precision %d", value);
    c->precision = value;
    return FH_OK;
  }
  if (option == FH_OPT_PREFETCH) {
    c->prefetch = value != 0;
    return FH_OK;
  }
  if (option == FH_OPT_SAMPLER) {
    if (value != FH_SAMPLER_EULER && value != FH_SAMPLER_RENOISE)
      return fail(c, FH_EINVAL, "unknown sampler %d", value);
    c->sampler = value;
    return FH_OK;
  }
  return fail(c, FH_EINVAL, "unknown option %d", option);
}

int fh_set_noise_seed(fh_ctx* c, uint64_t seed) {
  if (!c) return FH_EINVAL;
  c->noise_seed = seed;
  return FH_OK;
}

namespace {
// per block: ffn1 codes [Fd][D], ffn2 codes [D][Fd], then their scales
// [D/64][Fd] and [Fd/64][D] (uint16), each at a 256-byte boundary
size_t fp8_block_bytes(const fh_config& g) {
  auto r = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t D = g.dim, Fd = g.ffn_dim;
  return r(Fd * D) + r(D * Fd) + r(D / 64 * Fd * 2) + r(Fd / 64 * D * 2) + r(3 * D * D) + r(D / 64 * 3 * D * 2);
}
}  // namespace

size_t fh_fp8_weight_bytes(const fh_ctx* c) {
  if (!c) return 0;
  return fp8_block_bytes(c->cfg) * (size_t)c->cfg.n_blocks;
}

int fh_weights_quantize_fp8(fh_ctx* c, fh_weights* w, void* buf, size_t bytes, void* stream) {
  if (!c) return FH_EINVAL;
  if (!w || w->ctx != c) return fail(c, FH_EINVAL, "weights are null or bound to another context");
  if (!buf || ((uintptr_t)buf & 255)) return fail(c, FH_EINVAL, "buffer must be a non-null 256-byte aligned device pointer");
  if (bytes < fh_fp8_weight_bytes(c))
    return fail(c, FH_EINVAL, "buffer of %zu bytes is smaller than the %zu bytes needed", bytes, fh_fp8_weight_bytes(c));
  const fh_config& g = c->cfg;
  const int D = g.dim, Fd = g.ffn_dim;
  hipStream_t s = (hipStream_t)stream;
  auto r = [](size_t b) { return (b + 255) & ~(size_t)255; };
  char* p = (char*)buf;
  for (int i = 0; i < g.n_blocks; ++i) {
    WBlock& b = w->blk[i];
    uint8_t* q1 = (uint8_t*)p;
    uint8_t* q2 = q1 + r((size_t)Fd * D);
    uint16_t* s1 = (uint16_t*)(q2 + r((size_t)D * Fd));
    uint16_t* s2 = (uint16_t*)((char*)s1 + r((size_t)D / 64 * Fd * 2));
    uint8_t* q3 = (uint8_t*)((char*)s2 + r((size_t)Fd / 64 * D * 2));
    uint16_t* s3 = (uint16_t*)(q3 + r((size_t)3 * D * D));
    FH_HIP(fh::mx_quantize(nullptr, b.ffn1_w, Fd, D, q1, s1, s));
    FH_HIP(fh::mx_quantize(nullptr, b.ffn2_w, D, Fd, q2, s2, s));
    FH_HIP(fh::mx_quantize(nullptr, b.qkv_w, 3 * D, D, q3, s3, s));
    b.ffn1_q = q1; b.ffn1_s = s1; b.ffn2_q = q2; b.ffn2_s = s2; b.qkv_q = q3; b.qkv_s = s3;
    p += fp8_block_bytes(g);
  }
  w->fp8 = true;
  w->serial = g_weights_serial++;  // new FFN pointers: graphs captured before must not match
  return FH_OK;
}

int fh_mxfp8_quantize(const float* in, int64_t rows, int32_t K, uint8_t* codes, uint16_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 64) return FH_EINVAL;
  if (rows == 0) return FH_OK;
  if (!in || !codes || !scales || ((uintptr_t)in & 15) || ((uintptr_t)codes & 15) || ((uintptr_t)scales & 1))
    return FH_EINVAL;
  const hipError_t e = fh::mx_quantize(in, nullptr, rows, K, codes, scales, (hipStream_t)stream);
  return e == hipSuccess ? FH_OK : FH_EHIP;
}

int fh_mxfp8_gemm(const uint8_t* a, const uint16_t* a_scales, const uint8_t* w, const uint16_t* w_scales,
                  int64_t M, int32_t N, int32_t K, const float* bias, float* y, float* part, void* stream) {
  if (M < 0 || M > (1 << 24) || N <= 0 || N % 128 || K <= 0 || K % 64 || M % 2) return FH_EINVAL;
  if (M == 0) return FH_OK;
  auto al = [](const void* p, uintptr_t n) { return p && ((uintptr_t)p % n) == 0; };
  if (!al(a, 16) || !al(w, 16) || !al(a_scales, 4) || !al(w_scales, 4) || !al(bias, 16) || !al(y, 16) ||
      (part && !al(part, 16)))
    return FH_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (part) {
    if (!fh::gemm_splitk_ok((int)M, N, K)) return FH_EINVAL;
    e = fh::gemm_mx_splitk(a, K, a_scales, w, K, w_scales, (int)M, N, K, part, (size_t)2 * M * N, s);
    if (e == hipSuccess) {
      fh::PendingRes r;
      r.part = part;
      r.nparts = 2;
      r.bias = bias;
      e = fh::residual_from_parts(y, N, r, (int)M, N, s);
    }
  } else {
    fh::EpiArgs ep;
    ep.x = y;
    ep.ldx = N;
    ep.bias = bias;
    e = fh::gemm_mx(fh::EPI_RES, a, K, a_scales, w, K, w_scales, (int)M, N, K, ep, s);
  }
  return e == hipSuccess ? FH_OK : FH_EHIP;
}

int fh_philox4x32_fill(uint64_t seed, uint32_t lane, uint32_t step, uint32_t first_group, int64_t n_groups,
                       uint32_t* out, void* stream) {
  if (n_groups < 0 || (n_groups > 0 && !out) || ((uintptr_t)out & 15)) return FH_EINVAL;
  if (n_groups > 0 && (uint64_t)first_group + (uint64_t)(n_groups - 1) > 0xFFFFFFFFull) return FH_EINVAL;
  const hipError_t e = fh::philox_fill(out, n_groups, first_group, lane, step, seed, (hipStream_t)stream);
  return e == hipSuccess ? FH_OK : FH_EHIP;
}

namespace {
bool color_sizes_ok(int32_t F, int32_t H, int32_t W, int32_t Hr, int32_t Wr) {
  if (F < 0 || F > 65534 || H <= 0 || W <= 0 || Hr <= 0 || Wr <= 0) return false;
  const int64_t npix = (int64_t)H * W, nref = (int64_t)Hr * Wr;
  // the transfer launches up to one thread per frame pixel, and a launch
  // holds at most 2^32 - 1 work-items
  return npix <= (1ll << 32) && nref <= (1ll << 32) && (int64_t)F * npix <= (1ll << 32) - 256;
}
}  // namespace

size_t fh_color_match_workspace_bytes(int32_t n_frames, int32_t height, int32_t width, int32_t ref_height,
                                      int32_t ref_width) {
  if (!color_sizes_ok(n_frames, height, width, ref_height, ref_width) || n_frames == 0) return 0;
  return fh::color_match_workspace(n_frames, (int64_t)height * width, (int64_t)ref_height * ref_width);
}

int fh_color_match(const float* frames, int32_t n_frames, int32_t height, int32_t width, const float* picture,
                   int32_t ref_height, int32_t ref_width, float strength, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!color_sizes_ok(n_frames, height, width, ref_height, ref_width) || !std::isfinite(strength)) return FH_EINVAL;
  if (n_frames == 0) return FH_OK;
  if (!frames || !picture || !out || ((uintptr_t)frames & 3) || ((uintptr_t)picture & 3) || ((uintptr_t)out & 3))
    return FH_EINVAL;
  const int64_t npix = (int64_t)height * width, nref = (int64_t)ref_height * ref_width;
  const size_t bytes = (size_t)n_frames * npix * 3 * sizeof(float);
  if (out != frames && (const char*)out < (const char*)frames + bytes && (const char*)frames < (const char*)out + bytes)
    return FH_EINVAL;  // partial overlap
  const hipStream_t s = (hipStream_t)stream;
  if (strength == 0.0f) {  // correction disabled: the frames unchanged
    if (out == frames) return FH_OK;
    return hipMemcpyAsync(out, frames, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess ? FH_OK : FH_EHIP;
  }
  if (!workspace || ((uintptr_t)workspace & 255)) return FH_EINVAL;
  if (workspace_bytes < fh::color_match_workspace(n_frames, npix, nref)) return FH_EWORKSPACE;
  const hipError_t e = fh::color_match(frames, n_frames, npix, picture, nref, strength, out, workspace, s);
  return e == hipSuccess ? FH_OK : FH_EHIP;
}

int fh_color_match_noalloc(const float* frames, int32_t n_frames, int32_t height, int32_t width,
                           const float* picture, int32_t ref_height, int32_t ref_width, float strength, float* out,
                           void* stream) {
  if (!color_sizes_ok(n_frames, height, width, ref_height, ref_width) || !std::isfinite(strength)) return FH_EINVAL;
  if (n_frames == 0) return FH_OK;
  if (!frames || !picture || !out || ((uintptr_t)frames & 3) || ((uintptr_t)picture & 3) || ((uintptr_t)out & 3))
    return FH_EINVAL;
  const int64_t npix = (int64_t)height * width, nref = (int64_t)ref_height * ref_width;
  const size_t bytes = (size_t)n_frames * npix * 3 * sizeof(float);
  if (out != frames && (const char*)out < (const char*)frames + bytes && (const char*)frames < (const char*)out + bytes)
    return FH_EINVAL;  // partial overlap
  const hipStream_t s = (hipStream_t)stream;
  if (strength == 0.0f) {  // correction disabled: the frames unchanged
    if (out == frames) return FH_OK;
    return hipMemcpyAsync(out, frames, bytes, hipMemcpyDeviceToDevice, s) == hipSuccess ? FH_OK : FH_EHIP;
  }
  // the statistics of this call must fit the static scratch
  if (fh::color_match_workspace(n_frames, npix, nref) > fh::color_scratch_bytes()) return FH_EWORKSPACE;
  void* scratch = nullptr;
  if (fh::color_scratch(&scratch) != hipSuccess) return FH_EHIP;
  const hipError_t e = fh::color_match(frames, n_frames, npix, picture, nref, strength, out, scratch, s);
  return e == hipSuccess ? FH_OK : FH_EHIP;
}

size_t fh_color_match_noalloc_max_bytes(void) { return fh::color_scratch_bytes(); }

int fh_vae_weight_count(const fh_vae_config* v) { return vae_cfg_ok(v) ? (int)vae_specs(*v).size() : 0; }

int fh_vae_weight_spec(const fh_vae_config* v, int i, fh_tensor* out) {
  if (!out || !vae_cfg_ok(v)) return FH_EINVAL;
  static thread_local std::vector<Spec> specs;  // keeps the returned names alive until the next call
  specs = vae_specs(*v);
  if (i < 0 || i >= (int)specs.size()) return FH_EINVAL;
  std::memset(out, 0, sizeof *out);
  out->name = specs[i].name.c_str();
  out->dtype = specs[i].dtype;
  out->ndim = specs[i].ndim;
  out->shape[0] = specs[i].shape[0];
  out->shape[1] = specs[i].shape[1];
  return FH_OK;
}

int fh_vae_weights_bind(const fh_vae_config* v, const void* blob, size_t blob_bytes, const fh_tensor* index,
                        int n_index, fh_vae_weights** out) {
  if (!out) return FH_EINVAL;
  *out = nullptr;
  if (!vae_cfg_ok(v)) return FH_EINVAL;
  std::unordered_map<std::string, const void*> ptr;
  const int rc = resolve_tensors(nullptr, vae_specs(*v), blob, blob_bytes, index, n_index, ptr);
  if (rc) return rc;
  fh_vae_weights* w = new fh_vae_weights();
  w->cfg = *v;
  w->ptr = std::move(ptr);
  *out = w;
  return FH_OK;
}

void fh_vae_weights_release(fh_vae_weights* w) { delete w; }

size_t fh_vae_workspace_bytes(const fh_vae_config* v) { return vae_cfg_ok(v) ? carve_vae(*v, nullptr).total : 0; }

int fh_vae_decode(const fh_vae_weights* w, const float* latent, float* frames, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!w || !latent || !frames || ((uintptr_t)latent & 15) || ((uintptr_t)frames & 15)) return FH_EINVAL;
  const fh_vae_config& v = w->cfg;
  const VaeWS ws = carve_vae(v, (char*)workspace);
  if (!workspace || ((uintptr_t)workspace & 255)) return FH_EINVAL;
  if (workspace_bytes < ws.total) return FH_EWORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  auto P = [&](const std::string& n) { return w->ptr.at(n); };
  fh_ctx* c = nullptr;  // FH_HIP reports through c (none here)
  int T = v.frames, H = v.height, W = v.width;
  FH_HIP(fh::latent_to_f16(latent, v.latent_ch, (int64_t)T * H * W, ws.x0, ws.zero, s));
  auto conv = [&](int epi, const _Float16* in, int cin, const std::string& name, int cout, _Float16* out,
                  const _Float16* res, float* fr) {
    fh::ConvArgs a;
    a.in = in;
    a.T = T;
    a.H = H;
    a.W = W;
    a.cin_log2 = log2i(cin);
    a.w = (const _Float16*)P(name + ".w");
    a.bias = (const float*)P(name + ".b");
    a.cout = cout;
    a.zero = ws.zero;
    a.out = out;
    a.res = res;
    a.frames = fr;
    return fh::conv3d_f16(epi, a, ws.part, ws.part_elems, s);
  };
  FH_HIP(conv(fh::CONV_PLAIN, ws.x0, v.latent_ch, "conv_in", v.widths[0], ws.a, nullptr, nullptr));
  for (int i = 0; i < 3; ++i) {
    const std::string p = "up" + std::to_string(i) + ".";
    const int C = v.widths[i];
    const int64_t M = (int64_t)T * H * W;
    FH_HIP(fh::norm_silu_f16(ws.a, (const float*)P(p + "norm1.g"), ws.b, M, C, v.eps, s));
    FH_HIP(conv(fh::CONV_PLAIN, ws.b, C, p + "conv1", C, ws.c, nullptr, nullptr));
    FH_HIP(fh::norm_silu_f16(ws.c, (const float*)P(p + "norm2.g"), ws.b, M, C, v.eps, s));
    FH_HIP(conv(fh::CONV_RES, ws.b, C, p + "conv2", C, ws.c, ws.a, nullptr));
    FH_HIP(conv(fh::CONV_UP, ws.c, C, p + "up", 8 * v.widths[i + 1], ws.a, nullptr, nullptr));
    T = 2 * T - 1;
    H *= 2;
    W *= 2;
  }
  FH_HIP(fh::norm_silu_f16(ws.a, (const float*)P("norm_out.g"), ws.b, (int64_t)T * H * W, v.widths[3], v.eps, s));
  FH_HIP(conv(fh::CONV_FRAMES, ws.b, v.widths[3], "conv_out", v.out_ch * v.patch * v.patch, nullptr, nullptr,
              frames));
  return FH_OK;
}

int fh_audio_weight_count(const fh_ctx* c, const fh_audio_config* a) {
  if (!c || !a || check_audio_cfg(nullptr, a) != FH_OK) return 0;
  return (int)audio_specs(c, *a).size();
}

int fh_audio_weight_spec(const fh_ctx* c, const fh_audio_config* a, int i, fh_tensor* out) {
  if (!c || !a || !out) return FH_EINVAL;
  if (check_audio_cfg(nullptr, a) != FH_OK) return FH_EINVAL;
  static const char* const names[] = {"proj1.w", "proj1.b", "proj1vf.w", "proj1vf.b", "proj2.w",
                                      "proj2.b", "proj3.w", "proj3.b", "projNorm.g", "projNorm.b"};
  const std::vector<Spec> specs = audio_specs(c, *a);
  if (i < 0 || i >= (int)specs.size()) return FH_EINVAL;
  out->name = names[i];  // the same names as audio_specs, in its order (static storage)
  out->dtype = specs[i].dtype;
  out->ndim = specs[i].ndim;
  out->shape[0] = specs[i].shape[0];
  out->shape[1] = specs[i].shape[1];
  out->shape[2] = out->shape[3] = 0;
  out->offset = 0;
  return FH_OK;
}

int fh_audio_weights_bind(fh_ctx* c, const fh_audio_config* a, const void* blob, size_t blob_bytes,
                          const fh_tensor* index, int n_index, fh_audio_weights** out) {
  if (!c) return FH_EINVAL;
  if (!out) return fail(c, FH_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_audio_cfg(c, a);
  if (rc) return rc;
  std::unordered_map<std::string, const void*> ptr;
  rc = resolve_tensors(c, audio_specs(c, *a), blob, blob_bytes, index, n_index, ptr);
  if (rc) return rc;
  fh_audio_weights* w = new fh_audio_weights();
  w->serial = g_weights_serial++;
  w->ctx = c;
  w->acfg = *a;
  w->LF = c->cfg.frames;
  w->V = 1 + (c->cfg.frames - 1) * a->temporal_stride;
  w->F = a->window * a->layers * a->channels;
  auto M = [&](const char* n) { return (const bf16_t*)ptr[n]; };
  auto V = [&](const char* n) { return (const float*)ptr[n]; };
  w->p1_w = M("proj1.w"); w->p1_b = V("proj1.b");
  w->p1vf_w = M("proj1vf.w"); w->p1vf_b = V("proj1vf.b");
  w->p2_w = M("proj2.w"); w->p2_b = V("proj2.b");
  w->p3_w = M("proj3.w"); w->p3_b = V("proj3.b");
  w->norm_g = V("projNorm.g"); w->norm_b = V("projNorm.b");
  *out = w;
  return FH_OK;
}

void fh_audio_weights_release(fh_audio_weights* w) { delete w; }

size_t fh_audio_workspace_bytes(const fh_audio_weights* w, int batch) {
  if (!w || batch <= 0) return 0;
  return carve_audio(w, batch, nullptr).total;
}

int fh_audio_project(fh_ctx* c, const fh_audio_weights* w, int batch, const float* states, float* tokens,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!c) return FH_EINVAL;
  if (!w || w->ctx != c) return fail(c, FH_EINVAL, "audio weights are null or bound to another context");
  if (batch <= 0) return fail(c, FH_EINVAL, "batch must be positive, got %d", batch);
  if (!states || !tokens) return fail(c, FH_EINVAL, "null states or tokens");
  if (!ws || ((uintptr_t)ws & 255)) return fail(c, FH_EWORKSPACE, "workspace must be a non-null 256-byte aligned device pointer");
  const AudioWS a = carve_audio(w, batch, (char*)ws);
  if (ws_bytes < a.total)
    return fail(c, FH_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes batch %d needs", ws_bytes,
                a.total, batch);
  return enqueue_front(c, w, batch, states, a, tokens, nullptr, (hipStream_t)stream);
}

size_t fh_slice_from_states_workspace_bytes(const fh_ctx* c, const fh_audio_weights* w, int batch) {
  if (!c || !w || w->ctx != c || batch <= 0) return 0;
  return states_ws(c, w, batch, nullptr).total;
}

int fh_dit_denoise_slice_from_states(fh_ctx* c, const fh_weights* w, const fh_audio_weights* aw, int batch,
                                     const float* latent, const float* motion_latent, const float* states,
                                     const float* sigmas, int n_steps, float* latent_out, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!c) return FH_EINVAL;
  if (!aw || aw->ctx != c) return fail(c, FH_EINVAL, "audio weights are null or bound to another context");
  if (!states) return fail(c, FH_EINVAL, "null states");
  if (batch <= 0) return fail(c, FH_EINVAL, "batch must be positive, got %d", batch);
  if (!ws || ((uintptr_t)ws & 255))
    return fail(c, FH_EWORKSPACE, "workspace must be a non-null 256-byte aligned device pointer");
  const StatesWS sw = states_ws(c, aw, batch, (char*)ws);
  if (ws_bytes < sw.total)
    return fail(c, FH_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes batch %d needs", ws_bytes,
                sw.total, batch);
  FrontEnd fe{aw, states, sw.front, sw.tokens};
  return denoise_slice(c, w, batch, latent, motion_latent, nullptr, &fe, sigmas, n_steps, latent_out, sw.slice,
                       carve(c, batch, nullptr).total, stream);
}

int fh_debug_workgroup_order(int reversed) {
  if (reversed != 0 && reversed != 1) return FH_EINVAL;
  hipError_t (*const set[])(int) = {fh::set_wg_reverse_gemm, fh::set_wg_reverse_attn, fh::set_wg_reverse_color,
                                    fh::set_wg_reverse_norm, fh::set_wg_reverse_misc, fh::set_wg_reverse_vae};
  for (auto f : set)
    if (f(reversed) != hipSuccess) return FH_EHIP;
  return FH_OK;
}

int fh_shader_clock(void* dev_buf, size_t bytes, int n_wg, int iters, void* stream, double* mhz) {
  if (!dev_buf || !mhz || n_wg < 1 || n_wg > 65536 || iters < 1 || iters > (1 << 20) ||
      bytes < (size_t)32 * n_wg)
    return FH_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (fh::clock_probe((uint64_t*)dev_buf, n_wg, iters, s) != hipSuccess) return FH_EHIP;
  std::vector<uint64_t> h((size_t)4 * n_wg);
  if (hipMemcpyAsync(h.data(), dev_buf, h.size() * 8, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return FH_EHIP;
  int dev = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz <= 0)
    return FH_EHIP;
  std::vector<double> f;
  for (int i = 0; i < n_wg; ++i) {
    const uint64_t dt = h[4 * i + 1] - h[4 * i], dr = h[4 * i + 3] - h[4 * i + 2];
    if (dr > 0) f.push_back((double)dt / (double)dr * wall_khz / 1000.0);
  }
  if (f.empty()) return FH_EHIP;
  std::sort(f.begin(), f.end());
  *mhz = f[f.size() / 2];
  return FH_OK;
}

int fh_kernel_time(fh_ctx* c, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return FH_EINVAL;
  for (auto& e : c->ev_pending) {
    FH_HIP(hipEventSynchronize(e.second));
    float ms = 0.f;
    FH_HIP(hipEventElapsedTime(&ms, e.first, e.second));
    c->time_ms += ms;
    c->time_count += 1;
    c->ev_free.push_back(e);
  }
  c->ev_pending.clear();
  *total_ms = c->time_ms;
  *launches = c->time_count;
  c->time_ms = 0.0;
  c->time_count = 0;
  return FH_OK;
}

const char* fh_last_error(const fh_ctx* c) {
  if (!c) return "null context";
  return c->err.c_str();
}

const char* fh_status_str(int st) {
  switch (st) {
    case FH_OK: return "ok";
    case FH_EINVAL: return "invalid argument";
    case FH_ESHAPE: return "shape does not match the configuration";
    case FH_EUNSUPPORTED: return "configuration not implemented by the kernels";
    case FH_EWORKSPACE: return "workspace missing, misaligned or too small";
    case FH_EHIP: return "HIP runtime error";
    case FH_EWEIGHTS: return "weight tensor missing, misaligned or of the wrong dtype/shape";
    default: return "unknown status";
  }
}

}  // extern "C"
