// Host side of the KV-shared early-exit decoder: argument validation, buffer
// layouts, the layer scheduler for prefill and decode, and HIP-graph replay of
// decode steps.  Every decision of the method (the batch-minimum cosine against
// tau, the sticky exit flag) is taken on the device; the host only enqueues.
//
// Method: "River-LLM: Large Language Model Seamless Exit Based on KV Share"
// (section 3: shared-KV exit layers; section 4: exit rule; section 5:
// sequence-level exit in prefill, token-level exit in generation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "river_internal.h"

namespace river {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void linear_shapes(const river_config &c, LinearShape o[7]) {
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  o[0] = {qd, c.d_model};
  o[1] = {kd, c.d_model};
  o[2] = {kd, c.d_model};
  o[3] = {c.d_model, qd};
  o[4] = {c.ffn_dim, c.d_model};
  o[5] = {c.ffn_dim, c.d_model};
  o[6] = {c.d_model, c.ffn_dim};
}

static size_t linear_region(const river_config &c, const LinearShape &s, bool copy, size_t *sz_off) {
  if (copy) {
    *sz_off = 0;
    return align256((size_t)s.N * s.K * 2);
  }
  const size_t codes = align256((size_t)s.N * (s.K / 8) * 4);
  *sz_off = codes;
  return codes + align256((size_t)s.N * (s.K / c.group_size) * 4);
}

static size_t layer_region(const river_config &c, bool copy) {
  LinearShape sh[7];
  linear_shapes(c, sh);
  size_t t = 0, dummy;
  for (int i = 0; i < 7; ++i) t += linear_region(c, sh[i], copy, &dummy);
  return t;
}

void bank_offsets(const river_config &c, int layer, int linear, bool copy, size_t *codes, size_t *sz) {
  LinearShape sh[7];
  linear_shapes(c, sh);
  size_t off = (size_t)layer * layer_region(c, copy), szo = 0;
  for (int i = 0; i < linear; ++i) off += linear_region(c, sh[i], copy, &szo);
  linear_region(c, sh[linear], copy, &szo);
  *codes = off;
  *sz = copy ? 0 : off + szo;
}

// Decode steps of at least this many rows run RMSNorm and the exit test as
// row kernels and the normalised-input linears on the batched-row GEMM.
constexpr int kRowsPathMin = 5;


size_t bank_bytes(const river_config &c, bool copy) { return (size_t)c.n_layers * layer_region(c, copy); }

Workspace workspace_layout(const river_config &c) {
  Workspace w{};
  const int64_t R = (int64_t)c.max_batch * c.max_seq;
  const int qd = c.n_q_heads * c.head_dim;
  w.rows = R;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  w.hA = take((size_t)R * c.d_model * 4);
  w.hB = take((size_t)R * c.d_model * 4);
  w.x = take((size_t)R * c.d_model * 2);
  w.q = take((size_t)R * qd * 2);
  w.attn = take((size_t)R * qd * 2);
  w.u = take((size_t)R * c.ffn_dim * 2);
  const int64_t gemv_wgs = c.d_model / 4 + 1;
  const int64_t cos_wgs = (R + 3) / 4;
  w.part_floats = (int)std::max<int64_t>(gemv_wgs * kPartFloatsPerWG, cos_wgs);
  w.part = take((size_t)w.part_floats * 4);
  w.attn_splits = (c.max_seq + kAttnSub - 1) / kAttnSub;  // the most any batch size uses
  w.attn_part = take((size_t)c.max_batch * c.n_q_heads * w.attn_splits * (c.head_dim + 2) * 4);
  w.rope = take((size_t)c.max_seq * (c.head_dim / 2) * 8);
  // split-K partials of the batched-row GEMM (decode steps on the row-kernel path)
  int64_t mg = 0;
  if (c.max_batch >= kRowsPathMin) {
    const int kd = c.n_kv_heads * c.head_dim;
    const int shapes[5][2] = {{qd + 2 * kd, c.d_model}, {c.d_model, qd}, {2 * c.ffn_dim, c.d_model},
                              {c.d_model, c.ffn_dim}, {c.vocab, c.d_model}};
    const int rows[3] = {std::min(c.max_batch, 16), std::min(c.max_batch, 32), c.max_batch};
    for (int M : rows)
      for (auto &sh : shapes)
        mg = std::max<int64_t>(mg, mgemm_part_floats_max(M, sh[0], sh[1]));
  }
  w.mg_part_floats = std::max<int64_t>(mg, 1);
  w.mg_part = take((size_t)w.mg_part_floats * 4);
  // two K halves of the prefill GEMM's o and down outputs, up to 512 rows in
  // whole 64-row blocks
  w.pg_part_floats = 2 * ((std::min<int64_t>(R, 512) + 63) / 64) * 64 * c.d_model;
  w.pg_part = take((size_t)w.pg_part_floats * 4);
  w.total = off;
  return w;
}

// Offsets of the activation record of one pass with `rows` rows.
struct RecordLayout {
  size_t h_in, q, attn, h_mid, u, per_layer, h_out, total;
};
RecordLayout record_layout(const river_config &c, int64_t rows) {
  RecordLayout r{};
  const int64_t qd = (int64_t)c.n_q_heads * c.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  r.h_in = take(rows * c.d_model * 4);
  r.q = take(rows * qd * 2);
  r.attn = take(rows * qd * 2);
  r.h_mid = take(rows * c.d_model * 4);
  r.u = take(rows * c.ffn_dim * 2);
  r.per_layer = off;
  r.h_out = r.per_layer * c.n_layers;
  r.total = r.h_out + align256(rows * c.d_model * 4);
  return r;
}

}  // namespace river

using namespace river;

// ---------------------------------------------------------------------------
struct river_ctx {
  river_config cfg;
  std::vector<river_layer_w> layers;
  const uint16_t *embed, *final_norm, *lm_head;
  char *bank;
  size_t bank_size;
  uint16_t *kv;
  char *ws;
  Control *ctrl;
  hipStream_t stream;
  Workspace wl;
  bool built = false;
  int exit_mode = 0;
  int pos = 0;
  int batch = 0;
  bool use_graph = true;
  int force_E = -1;
  // One recorded decode step per (buffers, batch, forced E); tau is not part
  // of the key: a step reads it from the control block.
  struct GraphKey {
    const void *tok, *logits, *next;
    int B, force_E, steps;
    bool operator<(const GraphKey &o) const {
      return std::tie(tok, logits, next, B, force_E, steps) <
             std::tie(o.tok, o.logits, o.next, o.B, o.force_E, o.steps);
    }
  };
  std::map<GraphKey, hipGraphExec_t> graphs;
  // tau the control block holds (after a build it holds 0, a prefill writes
  // its own); a decode step with another tau first enqueues launch_set_tau
  uint32_t ctrl_tau_bits = 0;
  // profiling: events around every launch, folded into per-class totals on read
  bool profiling = false;
  struct Timed {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Timed> timed;
  std::vector<hipEvent_t> event_pool;
  // activation record (off when rec == nullptr)
  char *rec = nullptr;
  size_t rec_bytes = 0;
  int attn_chunk = 0;   // positions per decode-attention workgroup (0: chosen per shape)
  int gemv_mode = 0;    // RIVER_OPT_GEMV
  int attn_kind = 0;    // RIVER_OPT_ATTN
  std::vector<char> remote;   // per layer: backbone linears in host memory (offloaded)
  int strategy = kStratRiver; // RIVER_OPT_KV_STRATEGY
  // recompute comparator (one sequence): per position, its state at the
  // input of the first layer it holds no K/V for (caller-owned, fp32
  // [max_seq][d_model]), and that depth (non-increasing along the sequence)
  float *kv_state = nullptr;
  std::vector<int> depth;
};

namespace {

// recorded decode steps kept per context before the cache is emptied
constexpr size_t kMaxGraphs = 32;
constexpr int kMaxStepsPerCall = 64;   // decode steps one river_decode_steps call may take

bool valid_config(const river_config *c) {
  if (!c) return false;
  if (c->n_layers < 1 || c->n_layers > RIVER_MAX_LAYERS) return false;
  if (c->d_model < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->ffn_dim < 8 || c->vocab < 1 || c->group_size < 1 || c->max_batch < 1 || c->max_seq < 1)
    return false;
  if (!std::isfinite(c->rms_eps) || c->rms_eps < 0.f || !std::isfinite(c->rope_theta) ||
      c->rope_theta <= 0.f)
    return false;
  if (c->n_q_heads % c->n_kv_heads) return false;
  return true;
}

// shapes the kernels handle; RIVER_OK or RIVER_E_UNIMPLEMENTED
int supported(const river_config *c) {
  const int G = c->group_size;
  const int qd = c->n_q_heads * c->head_dim;
  if (G < 32 || G > 512 || (G & (G - 1))) return RIVER_E_UNIMPLEMENTED;
  if (c->d_model % G || c->ffn_dim % G || qd % G) return RIVER_E_UNIMPLEMENTED;
  if (c->d_model % 256 || c->ffn_dim % 256 || qd % 256) return RIVER_E_UNIMPLEMENTED;
  if (c->d_model > 8192) return RIVER_E_UNIMPLEMENTED;   // RMSNorm rows held in registers
  if (c->head_dim != 64 && c->head_dim != 128) return RIVER_E_UNIMPLEMENTED;
  const int gq = c->n_q_heads / c->n_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4) return RIVER_E_UNIMPLEMENTED;
  if (c->max_batch > 64) return RIVER_E_UNIMPLEMENTED;
  // more than 8 rows per decode step run on the batched-row MFMA GEMM
  if (c->max_batch >= kRowsPathMin && G != 64 && G != 128) return RIVER_E_UNIMPLEMENTED;
  if (c->ffn_dim % 32) return RIVER_E_UNIMPLEMENTED;
  return RIVER_OK;
}

template <class T>
T *at(char *base, size_t off) { return reinterpret_cast<T *>(base + off); }

void fill_weights(river_ctx *ctx, int l, int lin_first, int count, LinearWeights &w) {
  const river_layer_w &L = ctx->layers[l];
  const void *bb[7] = {L.wq, L.wk, L.wv, L.wo, L.w_gate, L.w_up, L.w_down};
  LinearShape sh[7];
  linear_shapes(ctx->cfg, sh);
  std::memset(&w, 0, sizeof(w));
  w.nseg = count;
  const bool copy = ctx->exit_mode == RIVER_EXIT_COPY;
  for (int i = 0; i < count; ++i) {
    const int lin = lin_first + i;
    w.bf[i] = static_cast<const uint16_t *>(bb[lin]);
    w.seg_rows[i] = sh[lin].N;
    size_t co, so;
    bank_offsets(ctx->cfg, l, lin, copy, &co, &so);
    if (copy) {
      w.ex_bf[i] = at<const uint16_t>(ctx->bank, co);
    } else {
      w.q4[i] = at<const uint32_t>(ctx->bank, co);
      w.sz[i] = at<const uint32_t>(ctx->bank, so);
    }
  }
}

uint16_t *k_layer(river_ctx *ctx, int l) {
  const river_config &c = ctx->cfg;
  return ctx->kv + (size_t)l * c.max_batch * c.n_kv_heads * c.max_seq * c.head_dim;
}
uint16_t *v_layer(river_ctx *ctx, int l) {
  const river_config &c = ctx->cfg;
  const size_t half = (size_t)c.n_layers * c.max_batch * c.n_kv_heads * c.max_seq * c.head_dim;
  return ctx->kv + half + (size_t)l * c.max_batch * c.n_kv_heads * c.max_seq * c.head_dim;
}

#define RV_TRY(expr)                         \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return RIVER_E_HIP; \
  } while (0)
#define RV_TRY_RC(expr)                 \
  do {                                  \
    const int rc_ = (expr);             \
    if (rc_ != RIVER_OK) return rc_;    \
  } while (0)

hipEvent_t take_event(river_ctx *ctx) {
  if (!ctx->event_pool.empty()) {
    hipEvent_t e = ctx->event_pool.back();
    ctx->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// When profiling, records an event before the launch and one after it (the
// interval holds the kernel and the dispatch gap in front of it).
struct TimedLaunch {
  river_ctx *ctx;
  int kind;
  hipEvent_t a = nullptr;
  TimedLaunch(river_ctx *c, int k) : ctx(c), kind(k) {
    if (ctx->profiling && (a = take_event(ctx))) (void)hipEventRecord(a, ctx->stream);
  }
  hipError_t done(hipError_t e) {
    if (a) {
      hipEvent_t b = take_event(ctx);
      if (b) {
        (void)hipEventRecord(b, ctx->stream);
        ctx->timed.push_back({kind, a, b});
      } else {
        ctx->event_pool.push_back(a);
      }
    }
    return e;
  }
};
#define TIMED(kind, expr) RV_TRY(TimedLaunch(ctx, kind).done(expr))
// Launch of one decode kernel class; with only >= 0 the others are skipped.
#define TIMED_ONLY(kind, expr) \
  if (only < 0 || only == (kind)) TIMED(kind, expr)

// Copy one produced array into the activation record (no-op when off).
struct Recorder {
  river_ctx *ctx;
  RecordLayout lay;
  int64_t rows;
  hipError_t put(int layer, size_t field, const void *src, size_t bytes) const {
    if (!ctx->rec) return hipSuccess;
    const size_t off = layer < 0 ? lay.h_out : layer * lay.per_layer + field;
    return hipMemcpyAsync(ctx->rec + off, src, bytes, hipMemcpyDeviceToDevice, ctx->stream);
  }
};

// Prefill GEMMs: the 128 x 128 tile kernel where its shape rules hold, the
// 64 x 64 one otherwise.
hipError_t launch_prefill_gemm(Epilogue ep, const GemmParams &g, hipStream_t s) {
  if (pgemm_fits(g.K, g.G)) return launch_pgemm(ep, g, s);
  return launch_gemm(ep, g, s);
}

// Common parameters of the batched-row GEMM launches of layer l.
GemmParams mgemm_base(river_ctx *ctx, int l, int M) {
  const river_config &c = ctx->cfg;
  GemmParams g{};
  g.M = M; g.G = c.group_size; g.layer = l; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl;
  g.Hq = c.n_q_heads; g.Hkv = c.n_kv_heads; g.Dh = c.head_dim; g.max_seq = c.max_seq;
  g.max_batch = c.max_batch; g.T = 0; g.rope_theta = c.rope_theta;
  g.rope = at<const float2>(ctx->ws, ctx->wl.rope);
  g.part = at<float>(ctx->ws, ctx->wl.mg_part);
  g.part_cap = ctx->wl.mg_part_floats;
  if (ctx->force_E >= 0 && l >= 0) g.path = l >= ctx->force_E ? kPathExit : kPathBackbone;
  return g;
}

// Final RMSNorm of B rows (row stride `stride` floats) + LM head + argmax on
// the batched-row GEMM.
int enqueue_lm_head_rows(river_ctx *ctx, const float *h, int64_t stride, int B, float *logits,
                         int32_t *next, int is_prefill) {
  const river_config &c = ctx->cfg;
  uint16_t *x = at<uint16_t>(ctx->ws, ctx->wl.x);
  RowsNormParams rn{h, x, ctx->final_norm, B, c.d_model, c.rms_eps, stride};
  TIMED(RIVER_K_P_NORM, launch_rows_norm(rn, ctx->stream));
  GemmParams lm = mgemm_base(ctx, -1, B);
  lm.w.bf[0] = ctx->lm_head; lm.w.seg_rows[0] = c.vocab; lm.w.nseg = 1;
  lm.N = c.vocab; lm.K = c.d_model; lm.x = x; lm.ldx = c.d_model;
  lm.logits = logits; lm.next = next; lm.vocab = c.vocab; lm.is_prefill = is_prefill;
  TIMED(RIVER_K_LMHEAD, launch_mgemm(kEpLogits, lm, ctx->stream));
  return RIVER_OK;
}

// Whether a decode step takes the row-kernel path (see below): always above 8
// rows; from kRowsPathMin rows unless a comparator other than the method
// itself runs, the backbone sits in host memory or a GEMV kind is forced
// (those keep the fused GEMVs up to 8 rows).
bool use_rows_path(const river_ctx *ctx) {
  if (ctx->batch > 8) return true;
  return ctx->batch >= kRowsPathMin && ctx->strategy == kStratRiver && ctx->gemv_mode == 0 &&
         std::none_of(ctx->remote.begin(), ctx->remote.end(), [](char r) { return r != 0; });
}

// Common fields of a decode GEMV of layer l over B rows.
GemvParams gemv_base(river_ctx *ctx, int l, int B) {
  const river_config &c = ctx->cfg;
  GemvParams g{};
  g.G = c.group_size; g.layer = l; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl; g.B = B;
  g.gemv_mode = ctx->gemv_mode;
  g.gshift = __builtin_ctz((unsigned)c.group_size);
  g.eps = c.rms_eps; g.Hq = c.n_q_heads; g.Hkv = c.n_kv_heads; g.Dh = c.head_dim;
  g.max_seq = c.max_seq; g.max_batch = c.max_batch; g.rope_theta = c.rope_theta;
  g.rope = at<const float2>(ctx->ws, ctx->wl.rope);
  g.n_layers = c.n_layers;
  // a forced exit layer fixes every weight choice on the host: no kernel
  // then waits for the device flag before streaming its weights
  if (ctx->force_E >= 0 && l >= 0) g.path = l >= ctx->force_E ? kPathExit : kPathBackbone;
  return g;
}

// Final RMSNorm + LM head + argmax of B <= 8 decode rows on the GEMV.
int enqueue_lm_head_gemv(river_ctx *ctx, const float *h, int B, float *logits, int32_t *next,
                         hipStream_t s) {
  const river_config &c = ctx->cfg;
  GemvParams lm{};
  lm.w.bf[0] = ctx->lm_head; lm.w.seg_rows[0] = c.vocab; lm.w.nseg = 1;
  lm.gemv_mode = ctx->gemv_mode;
  lm.N = c.vocab; lm.K = c.d_model; lm.G = c.group_size; lm.layer = -1;
  lm.gshift = __builtin_ctz((unsigned)c.group_size);
  lm.exit_mode = ctx->exit_mode; lm.ctrl = ctx->ctrl; lm.B = B;
  lm.h_src = h; lm.h_stride = c.d_model; lm.gain = ctx->final_norm; lm.eps = c.rms_eps;
  lm.logits = logits; lm.next = next; lm.is_prefill = 0; lm.vocab = c.vocab;
  TIMED(RIVER_K_LMHEAD, launch_gemv(kXNorm, kEpLogits, lm, s));
  return RIVER_OK;
}

// Decode step on row kernels: RMSNorm and the exit test as row kernels (the
// test is the same batch-min rule; its flag is read by the next layer's
// GEMMs), the linears with normalised inputs (q|k|v, gate|up) on the
// batched-row MFMA GEMM.  More than 8 rows: o and down there too.  5..8 rows
// (kRowsPathMin): o and down on the matrix-core GEMV with the bf16 rows
// through its load ring, and the LM head on the GEMV; normalising the rows
// once per layer here beats staging them normalised in every workgroup of
// the fused GEMVs (8B shape, 8 rows: q|k|v 26.0 -> 14.5 us, gate|up 35.3 ->
// 29.5 us), while o and down stay faster on the GEMV.
int enqueue_decode_rows(river_ctx *ctx, const int32_t *tok, float tau, float *logits, int32_t *next,
                        int only) {
  const river_config &c = ctx->cfg;
  const int B = ctx->batch;
  const bool few = B <= 8;
  hipStream_t s = ctx->stream;
  float *hA = at<float>(ctx->ws, ctx->wl.hA), *hB = at<float>(ctx->ws, ctx->wl.hB);
  uint16_t *x = at<uint16_t>(ctx->ws, ctx->wl.x);
  const int qd = c.n_q_heads * c.head_dim;
  const Recorder rec{ctx, record_layout(c, B), B};
  const size_t hbytes = (size_t)B * c.d_model * 4, qbytes = (size_t)B * qd * 2;

  BeginParams bp{};
  bp.ctrl = ctx->ctrl; bp.tokens = tok; bp.rows = B; bp.B = B; bp.embed = ctx->embed; bp.h = hA;
  bp.d = c.d_model; bp.vocab = c.vocab; bp.n_layers = c.n_layers; bp.force_E = ctx->force_E;
  bp.tau = tau; bp.write_tau = 0; bp.is_prefill = 0; bp.set_pos = -1; bp.strategy = ctx->strategy;
  TIMED_ONLY(RIVER_K_BEGIN, launch_begin(bp, s));

  for (int l = 0; l < c.n_layers; ++l) {
    const river_layer_w &L = ctx->layers[l];
    RV_TRY(rec.put(l, rec.lay.h_in, hA, hbytes));
    if (l == 0) {
      // (deeper layers get their normalised rows from the previous layer's
      // last launch, together with its exit test)
      RowsNormParams rn{hA, x, static_cast<const uint16_t *>(L.attn_norm), B, c.d_model, c.rms_eps, 0};
      TIMED_ONLY(RIVER_K_P_NORM, launch_rows_norm(rn, s));
    }

    GemmParams q = mgemm_base(ctx, l, B);
    fill_weights(ctx, l, 0, 3, q.w);
    q.N = qd + 2 * c.n_kv_heads * c.head_dim; q.K = c.d_model; q.x = x; q.ldx = c.d_model;
    q.q_out = at<uint16_t>(ctx->ws, ctx->wl.q);
    q.k_cache = k_layer(ctx, l); q.v_cache = v_layer(ctx, l);
    TIMED_ONLY(RIVER_K_QKV, launch_mgemm(kEpQKV, q, s));
    RV_TRY(rec.put(l, rec.lay.q, q.q_out, qbytes));

    AttnParams a{};
    a.q = q.q_out; a.k_cache = q.k_cache; a.v_cache = q.v_cache;
    a.out = at<uint16_t>(ctx->ws, ctx->wl.attn); a.part = at<float>(ctx->ws, ctx->wl.attn_part);
    a.counters = control_attn_counters(ctx->ctrl, c.max_batch); a.ctrl = ctx->ctrl;
    a.B = B; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.Dh = c.head_dim; a.S = c.max_seq;
    a.chunk = ctx->attn_chunk > 0 ? ctx->attn_chunk : attn_chunk(c.max_seq, B, c.n_kv_heads);
    a.splits = (c.max_seq + a.chunk - 1) / a.chunk;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    a.mfma = ctx->attn_kind == 0;
    a.layer = l;
    a.pos_E = ctx->strategy == kStratMask ? control_pos_E(ctx->ctrl, c.max_batch, c.n_kv_heads) : nullptr;
    a.nw8 = a.mfma && a.splits == 1 && a.chunk % (2 * kAttnSub) == 0;
    TIMED_ONLY(RIVER_K_ATTN, launch_attn_decode(a, s));
    RV_TRY(rec.put(l, rec.lay.attn, a.out, qbytes));

    if (few) {
      GemvParams o = gemv_base(ctx, l, B);
      fill_weights(ctx, l, 3, 1, o.w);
      o.N = c.d_model; o.K = qd; o.x_src = a.out; o.x_stride = qd;
      o.h_in = hA; o.h_out = hB; o.h_io_stride = c.d_model;
      TIMED_ONLY(RIVER_K_O, launch_gemv(kXBf16, kEpResid, o, s));
    } else {
      GemmParams o = mgemm_base(ctx, l, B);
      fill_weights(ctx, l, 3, 1, o.w);
      o.N = c.d_model; o.K = qd; o.x = a.out; o.ldx = qd;
      o.h_in = hA; o.h_out = hB; o.h_io_stride = c.d_model;
      TIMED_ONLY(RIVER_K_O, launch_mgemm(kEpResid, o, s));
    }
    RV_TRY(rec.put(l, rec.lay.h_mid, hB, hbytes));

    RowsNormParams rn2{hB, x, static_cast<const uint16_t *>(L.mlp_norm), B, c.d_model, c.rms_eps, 0};
    TIMED_ONLY(RIVER_K_P_NORM, launch_rows_norm(rn2, s));
    GemmParams gu = mgemm_base(ctx, l, B);
    fill_weights(ctx, l, 4, 2, gu.w);
    gu.N = 2 * c.ffn_dim; gu.K = c.d_model; gu.x = x; gu.ldx = c.d_model;
    gu.u_out = at<uint16_t>(ctx->ws, ctx->wl.u);
    TIMED_ONLY(RIVER_K_GATEUP, launch_mgemm(kEpSwiGLU, gu, s));
    RV_TRY(rec.put(l, rec.lay.u, gu.u_out, (size_t)B * c.ffn_dim * 2));

    if (few) {
      GemvParams dn = gemv_base(ctx, l, B);
      fill_weights(ctx, l, 6, 1, dn.w);
      dn.N = c.d_model; dn.K = c.ffn_dim; dn.x_src = gu.u_out; dn.x_stride = c.ffn_dim;
      dn.h_in = hB; dn.h_out = hB; dn.h_io_stride = c.d_model;
      TIMED_ONLY(RIVER_K_DOWN, launch_gemv(kXBf16, kEpResid, dn, s));
    } else {
      GemmParams dn = mgemm_base(ctx, l, B);
      fill_weights(ctx, l, 6, 1, dn.w);
      dn.N = c.d_model; dn.K = c.ffn_dim; dn.x = gu.u_out; dn.ldx = c.ffn_dim;
      dn.h_in = hB; dn.h_out = hB; dn.h_io_stride = c.d_model;
      TIMED_ONLY(RIVER_K_DOWN, launch_mgemm(kEpResid, dn, s));
    }

    if (l < c.n_layers - 1) {
      // the exit test after this layer and the next layer's input RMSNorm
      RowsCosParams rc{hA, hB, B, c.d_model, at<float>(ctx->ws, ctx->wl.part), ctx->ctrl, l,
                       c.n_layers};
      RowsNormParams rn{hB, x, static_cast<const uint16_t *>(ctx->layers[l + 1].attn_norm), B, c.d_model,
                        c.rms_eps, 0};
      TIMED_ONLY(RIVER_K_P_COS, launch_rows_cos_norm(rc, rn, ctx->force_E < 0, s));
    }
    std::swap(hA, hB);
  }
  RV_TRY(rec.put(-1, 0, hA, hbytes));
  if (only < 0 && few) return enqueue_lm_head_gemv(ctx, hA, B, logits, next, s);
  if (only < 0) return enqueue_lm_head_rows(ctx, hA, c.d_model, B, logits, next, 0);
  return RIVER_OK;
}

// Recompute comparator: layer l (backbone) for the n earlier positions
// q0 .. q0+n-1 that hold no K/V at l, as rows of one prefill-style pass
// (positions offset by q0, causal attention over the cache), their states
// read from and written back to kv_state.  Every launch does nothing once
// the current pass is past its exit at l.  Rows 1.. of the workspace (row 0
// is the current token's).
int enqueue_pending_rows(river_ctx *ctx, int l, int q0, int n) {
  const river_config &c = ctx->cfg;
  hipStream_t s = ctx->stream;
  const river_layer_w &L = ctx->layers[l];
  const int qd = c.n_q_heads * c.head_dim;
  float *H = ctx->kv_state + (int64_t)q0 * c.d_model;
  float *hC = at<float>(ctx->ws, ctx->wl.hB) + c.d_model;
  uint16_t *x = at<uint16_t>(ctx->ws, ctx->wl.x) + c.d_model;
  GemmParams g{};
  g.M = n; g.G = c.group_size; g.layer = l; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl;
  g.Hq = c.n_q_heads; g.Hkv = c.n_kv_heads; g.Dh = c.head_dim; g.max_seq = c.max_seq;
  g.max_batch = c.max_batch; g.T = n; g.start = q0; g.rope_theta = c.rope_theta;
  g.rope = at<const float2>(ctx->ws, ctx->wl.rope);
  g.path = kPathPending;

  RowsNormParams rn{H, x, static_cast<const uint16_t *>(L.attn_norm), n, c.d_model, c.rms_eps, 0,
                    ctx->ctrl, l, kPathPending};
  TIMED(RIVER_K_P_NORM, launch_rows_norm(rn, s));
  GemmParams q = g;
  fill_weights(ctx, l, 0, 3, q.w);
  q.N = qd + 2 * c.n_kv_heads * c.head_dim; q.K = c.d_model; q.x = x; q.ldx = c.d_model;
  q.q_out = at<uint16_t>(ctx->ws, ctx->wl.q) + qd;
  q.k_cache = k_layer(ctx, l); q.v_cache = v_layer(ctx, l);
  TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpQKV, q, s));

  AttnPrefillParams ap{};
  ap.q = q.q_out; ap.k_cache = q.k_cache; ap.v_cache = q.v_cache;
  ap.out = at<uint16_t>(ctx->ws, ctx->wl.attn) + qd; ap.B = 1; ap.T = n; ap.start = q0;
  ap.Hq = c.n_q_heads; ap.Hkv = c.n_kv_heads; ap.Dh = c.head_dim; ap.S = c.max_seq;
  ap.scale = 1.0f / std::sqrt((float)c.head_dim);
  ap.mfma = ctx->attn_kind == 0;
  ap.ctrl = ctx->ctrl; ap.layer = l; ap.path = kPathPending;
  TIMED(RIVER_K_P_ATTN, launch_attn_prefill(ap, s));

  GemmParams o = g;
  fill_weights(ctx, l, 3, 1, o.w);
  o.N = c.d_model; o.K = qd; o.x = ap.out; o.ldx = qd;
  o.h_in = H; o.h_out = hC; o.h_io_stride = c.d_model;
  TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpResid, o, s));
  RowsNormParams rn2{hC, x, static_cast<const uint16_t *>(L.mlp_norm), n, c.d_model, c.rms_eps, 0,
                     ctx->ctrl, l, kPathPending};
  TIMED(RIVER_K_P_NORM, launch_rows_norm(rn2, s));
  GemmParams gu = g;
  fill_weights(ctx, l, 4, 2, gu.w);
  gu.N = 2 * c.ffn_dim; gu.K = c.d_model; gu.x = x; gu.ldx = c.d_model;
  gu.u_out = at<uint16_t>(ctx->ws, ctx->wl.u) + c.ffn_dim;
  TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpSwiGLU, gu, s));
  GemmParams dn = g;
  fill_weights(ctx, l, 6, 1, dn.w);
  dn.N = c.d_model; dn.K = c.ffn_dim; dn.x = gu.u_out; dn.ldx = c.ffn_dim;
  dn.h_in = hC; dn.h_out = hC; dn.h_io_stride = c.d_model;
  TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpResid, dn, s));
  RV_TRY(launch_rows_copy_run(H, hC, (int64_t)n * c.d_model, ctx->ctrl, l, kPathPending, s));
  return RIVER_OK;
}

// Enqueue one decode step (B <= 8 rows): GEMV linears + split-K attention.
//
// only >= 0 (a RIVER_K_* layer kernel class) enqueues nothing but that class's
// launch for every layer, with the same parameters (kernel timing).
int enqueue_decode(river_ctx *ctx, const int32_t *tok, float tau, float *logits, int32_t *next,
                   int only = -1) {
  if (use_rows_path(ctx)) return enqueue_decode_rows(ctx, tok, tau, logits, next, only);
  const river_config &c = ctx->cfg;
  const int B = ctx->batch;
  hipStream_t s = ctx->stream;
  float *hA = at<float>(ctx->ws, ctx->wl.hA), *hB = at<float>(ctx->ws, ctx->wl.hB);
  const int qd = c.n_q_heads * c.head_dim;
  const Recorder rec{ctx, record_layout(c, B), B};
  const size_t hbytes = (size_t)B * c.d_model * 4, qbytes = (size_t)B * qd * 2;

  BeginParams bp{};
  bp.ctrl = ctx->ctrl; bp.tokens = tok; bp.rows = B; bp.B = B; bp.embed = ctx->embed; bp.h = hA;
  bp.d = c.d_model; bp.vocab = c.vocab; bp.n_layers = c.n_layers; bp.force_E = ctx->force_E;
  bp.tau = tau; bp.write_tau = 0; bp.is_prefill = 0; bp.set_pos = -1; bp.strategy = ctx->strategy;
  TIMED_ONLY(RIVER_K_BEGIN, launch_begin(bp, s));

  int down_wgs = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    const river_layer_w &L = ctx->layers[l];
    GemvParams g{};
    g.G = c.group_size; g.layer = l; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl; g.B = B;
    g.gemv_mode = ctx->gemv_mode;
    g.gshift = __builtin_ctz((unsigned)c.group_size);
    g.eps = c.rms_eps; g.Hq = c.n_q_heads; g.Hkv = c.n_kv_heads; g.Dh = c.head_dim;
    g.max_seq = c.max_seq; g.max_batch = c.max_batch; g.rope_theta = c.rope_theta;
    g.rope = at<const float2>(ctx->ws, ctx->wl.rope);
    g.n_layers = c.n_layers;
    // a forced exit layer fixes every weight choice on the host: no kernel
    // then waits for the device flag before streaming its weights
    if (ctx->force_E >= 0) g.path = l >= ctx->force_E ? kPathExit : kPathBackbone;

    // attention RMSNorm + fused q|k|v + RoPE + write into the shared slot
    GemvParams q = g;
    fill_weights(ctx, l, 0, 3, q.w);
    q.N = qd + 2 * c.n_kv_heads * c.head_dim; q.K = c.d_model;
    q.h_src = hA; q.h_stride = c.d_model; q.gain = static_cast<const uint16_t *>(L.attn_norm);
    q.q_out = at<uint16_t>(ctx->ws, ctx->wl.q);
    q.k_cache = k_layer(ctx, l); q.v_cache = v_layer(ctx, l);
    // the exit test after layer l-1 is decided at the start of this kernel
    q.test_prev = l > 0; q.part = at<float>(ctx->ws, ctx->wl.part); q.part_wgs = down_wgs;
    q.remote_bb = ctx->remote.empty() ? 0 : ctx->remote[l];
    RV_TRY(rec.put(l, rec.lay.h_in, hA, hbytes));
    TIMED_ONLY(RIVER_K_QKV, launch_gemv(kXNorm, kEpQKV, q, s));
    RV_TRY(rec.put(l, rec.lay.q, q.q_out, qbytes));
    if (ctx->strategy == kStratRecompute && only < 0) {
      // (this layer's exit decision is taken by now: the launch above made it)
      const int pos = ctx->pos;
      const int q0 = (int)(std::partition_point(ctx->depth.begin(), ctx->depth.begin() + pos,
                                                [l](int d) { return d > l; }) - ctx->depth.begin());
      // (with the exit forced the host knows which layers run)
      if (q0 < pos && (ctx->force_E < 0 || l < ctx->force_E))
        RV_TRY_RC(enqueue_pending_rows(ctx, l, q0, pos - q0));
    }

    AttnParams a{};
    a.q = q.q_out; a.k_cache = q.k_cache; a.v_cache = q.v_cache;
    a.out = at<uint16_t>(ctx->ws, ctx->wl.attn); a.part = at<float>(ctx->ws, ctx->wl.attn_part);
    a.counters = control_attn_counters(ctx->ctrl, c.max_batch); a.ctrl = ctx->ctrl;
    a.B = B; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.Dh = c.head_dim; a.S = c.max_seq;
    a.chunk = ctx->attn_chunk > 0 ? ctx->attn_chunk : attn_chunk(c.max_seq, B, c.n_kv_heads);
    a.splits = (c.max_seq + a.chunk - 1) / a.chunk;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    a.mfma = ctx->attn_kind == 0;
    a.layer = l;
    a.pos_E = ctx->strategy == kStratMask ? control_pos_E(ctx->ctrl, c.max_batch, c.n_kv_heads) : nullptr;
    a.nw8 = a.mfma && a.splits == 1 && a.chunk % (2 * kAttnSub) == 0;
    TIMED_ONLY(RIVER_K_ATTN, launch_attn_decode(a, s));
    RV_TRY(rec.put(l, rec.lay.attn, a.out, qbytes));

    GemvParams o = g;
    fill_weights(ctx, l, 3, 1, o.w);
    o.N = c.d_model; o.K = qd; o.x_src = a.out; o.x_stride = qd;
    o.h_in = hA; o.h_out = hB; o.h_io_stride = c.d_model;
    TIMED_ONLY(RIVER_K_O, launch_gemv(kXBf16, kEpResid, o, s));
    RV_TRY(rec.put(l, rec.lay.h_mid, hB, hbytes));

    GemvParams gu = g;
    fill_weights(ctx, l, 4, 2, gu.w);
    gu.N = 2 * c.ffn_dim; gu.K = c.d_model;
    gu.h_src = hB; gu.h_stride = c.d_model; gu.gain = static_cast<const uint16_t *>(L.mlp_norm);
    gu.u_out = at<uint16_t>(ctx->ws, ctx->wl.u); gu.u_stride = c.ffn_dim;
    TIMED_ONLY(RIVER_K_GATEUP, launch_gemv(kXNorm, kEpSwiGLU, gu, s));
    RV_TRY(rec.put(l, rec.lay.u, gu.u_out, (size_t)B * c.ffn_dim * 2));

    GemvParams dn = g;
    fill_weights(ctx, l, 6, 1, dn.w);
    dn.N = c.d_model; dn.K = c.ffn_dim; dn.x_src = gu.u_out; dn.x_stride = c.ffn_dim;
    dn.h_in = hB; dn.h_out = hB; dn.h_io_stride = c.d_model; dn.h_src = hA;
    dn.part = at<float>(ctx->ws, ctx->wl.part);
    dn.test_exit = l < c.n_layers - 1;
    down_wgs = gemv_grid(kEpResidExit, dn);
    TIMED_ONLY(RIVER_K_DOWN, launch_gemv(kXBf16, kEpResidExit, dn, s));
    std::swap(hA, hB);
  }
  RV_TRY(rec.put(-1, 0, hA, hbytes));
  if (only < 0) RV_TRY_RC(enqueue_lm_head_gemv(ctx, hA, B, logits, next, s));
  if (ctx->strategy == kStratMask && only < 0)
    RV_TRY(launch_set_pos_E(ctx->ctrl, control_pos_E(ctx->ctrl, c.max_batch, c.n_kv_heads), 0, s));
  if (ctx->strategy == kStratRecompute && only < 0)   // this position's state at its exit
    RV_TRY(hipMemcpyAsync(ctx->kv_state + (int64_t)ctx->pos * c.d_model, hA, (size_t)c.d_model * 4,
                          hipMemcpyDeviceToDevice, s));
  return RIVER_OK;
}

int enqueue_prefill(river_ctx *ctx, const int32_t *tok, int B, int T, float tau, float *logits,
                    int32_t *next) {
  const river_config &c = ctx->cfg;
  hipStream_t s = ctx->stream;
  const int64_t R = (int64_t)B * T;
  float *hA = at<float>(ctx->ws, ctx->wl.hA), *hB = at<float>(ctx->ws, ctx->wl.hB);
  uint16_t *x = at<uint16_t>(ctx->ws, ctx->wl.x);
  const int qd = c.n_q_heads * c.head_dim;
  const Recorder rec{ctx, record_layout(c, R), R};
  const size_t hbytes = (size_t)R * c.d_model * 4, qbytes = (size_t)R * qd * 2;

  BeginParams bp{};
  bp.ctrl = ctx->ctrl; bp.tokens = tok; bp.rows = R; bp.B = B; bp.embed = ctx->embed; bp.h = hA;
  bp.d = c.d_model; bp.vocab = c.vocab; bp.n_layers = c.n_layers; bp.force_E = ctx->force_E;
  bp.tau = tau; bp.write_tau = 1; bp.is_prefill = 1; bp.set_pos = T; bp.strategy = ctx->strategy;
  TIMED(RIVER_K_BEGIN, launch_begin(bp, s));

  for (int l = 0; l < c.n_layers; ++l) {
    const river_layer_w &L = ctx->layers[l];
    GemmParams g{};
    g.M = (int)R; g.G = c.group_size; g.layer = l; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl;
    g.Hq = c.n_q_heads; g.Hkv = c.n_kv_heads; g.Dh = c.head_dim; g.max_seq = c.max_seq;
    g.max_batch = c.max_batch; g.T = T; g.rope_theta = c.rope_theta;
    g.rope = at<const float2>(ctx->ws, ctx->wl.rope);
    if (ctx->force_E >= 0) g.path = l >= ctx->force_E ? kPathExit : kPathBackbone;

    RV_TRY(rec.put(l, rec.lay.h_in, hA, hbytes));
    RowsNormParams rn{hA, x, static_cast<const uint16_t *>(L.attn_norm), R, c.d_model, c.rms_eps, 0,
                      ctx->ctrl, l, g.path};
    TIMED(RIVER_K_P_NORM, launch_rows_norm(rn, s));

    GemmParams q = g;
    fill_weights(ctx, l, 0, 3, q.w);
    q.N = qd + 2 * c.n_kv_heads * c.head_dim; q.K = c.d_model; q.x = x; q.ldx = c.d_model;
    q.q_out = at<uint16_t>(ctx->ws, ctx->wl.q);
    q.k_cache = k_layer(ctx, l); q.v_cache = v_layer(ctx, l);
    TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpQKV, q, s));
    RV_TRY(rec.put(l, rec.lay.q, q.q_out, qbytes));

    AttnPrefillParams ap{};
    ap.q = q.q_out; ap.k_cache = q.k_cache; ap.v_cache = q.v_cache;
    ap.out = at<uint16_t>(ctx->ws, ctx->wl.attn); ap.B = B; ap.T = T; ap.Hq = c.n_q_heads;
    ap.Hkv = c.n_kv_heads; ap.Dh = c.head_dim; ap.S = c.max_seq;
    ap.scale = 1.0f / std::sqrt((float)c.head_dim);
    ap.mfma = ctx->attn_kind == 0;
    ap.ctrl = ctx->ctrl; ap.layer = l; ap.path = g.path;
    TIMED(RIVER_K_P_ATTN, launch_attn_prefill(ap, s));
    RV_TRY(rec.put(l, rec.lay.attn, ap.out, qbytes));

    GemmParams o = g;
    fill_weights(ctx, l, 3, 1, o.w);
    o.N = c.d_model; o.K = qd; o.x = ap.out; o.ldx = qd;
    o.h_in = hA; o.h_out = hB; o.h_io_stride = c.d_model;
    o.part = at<float>(ctx->ws, ctx->wl.pg_part); o.part_cap = ctx->wl.pg_part_floats;
    TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpResid, o, s));
    RV_TRY(rec.put(l, rec.lay.h_mid, hB, hbytes));

    RowsNormParams rn2{hB, x, static_cast<const uint16_t *>(L.mlp_norm), R, c.d_model, c.rms_eps, 0,
                       ctx->ctrl, l, g.path};
    TIMED(RIVER_K_P_NORM, launch_rows_norm(rn2, s));

    GemmParams gu = g;
    fill_weights(ctx, l, 4, 2, gu.w);
    gu.N = 2 * c.ffn_dim; gu.K = c.d_model; gu.x = x; gu.ldx = c.d_model;
    gu.u_out = at<uint16_t>(ctx->ws, ctx->wl.u);
    TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpSwiGLU, gu, s));
    RV_TRY(rec.put(l, rec.lay.u, gu.u_out, (size_t)R * c.ffn_dim * 2));

    GemmParams dn = g;
    fill_weights(ctx, l, 6, 1, dn.w);
    dn.N = c.d_model; dn.K = c.ffn_dim; dn.x = gu.u_out; dn.ldx = c.ffn_dim;
    dn.h_in = hB; dn.h_out = hB; dn.h_io_stride = c.d_model;
    dn.part = o.part; dn.part_cap = o.part_cap;
    TIMED(RIVER_K_P_GEMM, launch_prefill_gemm(kEpResid, dn, s));

    if (l < c.n_layers - 1 && ctx->force_E < 0) {
      RowsCosParams rc{hA, hB, R, c.d_model, at<float>(ctx->ws, ctx->wl.part), ctx->ctrl, l,
                       c.n_layers};
      TIMED(RIVER_K_P_COS, launch_rows_cos_exit(rc, s));
    }
    std::swap(hA, hB);
  }
  RV_TRY(rec.put(-1, 0, hA, hbytes));
  if (ctx->strategy == kStratRecompute)   // (one sequence) every prompt position's state at the exit
    RV_TRY(hipMemcpyAsync(ctx->kv_state, hA, (size_t)T * c.d_model * 4, hipMemcpyDeviceToDevice, s));
  if (B > 8) {
    const int st = enqueue_lm_head_rows(ctx, hA + (int64_t)(T - 1) * c.d_model, (int64_t)T * c.d_model, B,
                                        logits, next, 1);
    if (st != RIVER_OK) return st;
    // (kv mask: every prompt position holds K/V up to the prompt's exit)
    if (ctx->strategy == kStratMask)
      RV_TRY(launch_set_pos_E(ctx->ctrl, control_pos_E(ctx->ctrl, c.max_batch, c.n_kv_heads), T, s));
    return RIVER_OK;
  }
  GemvParams lm{};
  lm.w.bf[0] = ctx->lm_head; lm.w.seg_rows[0] = c.vocab; lm.w.nseg = 1;
  lm.gemv_mode = ctx->gemv_mode;
  lm.N = c.vocab; lm.K = c.d_model; lm.G = c.group_size; lm.layer = -1;
  lm.gshift = __builtin_ctz((unsigned)c.group_size);
  lm.exit_mode = ctx->exit_mode; lm.ctrl = ctx->ctrl; lm.B = B;
  lm.h_src = hA + (int64_t)(T - 1) * c.d_model; lm.h_stride = (int64_t)T * c.d_model;
  lm.gain = ctx->final_norm; lm.eps = c.rms_eps;
  lm.logits = logits; lm.next = next; lm.is_prefill = 1; lm.vocab = c.vocab;
  TIMED(RIVER_K_LMHEAD, launch_gemv(kXNorm, kEpLogits, lm, s));
  if (ctx->strategy == kStratMask)
    RV_TRY(launch_set_pos_E(ctx->ctrl, control_pos_E(ctx->ctrl, c.max_batch, c.n_kv_heads), T, s));
  return RIVER_OK;
}

// Recompute comparator: the pass just enqueued exited at E (read back: the
// next pass's launches depend on it); positions up to `last` hold at least
// E layers now, `first` .. `last` exactly E if they held fewer.
int note_depth(river_ctx *ctx, int first, int last) {
  int32_t E = 0;
  RV_TRY(hipMemcpyAsync(&E, &ctx->ctrl->last_E, sizeof(E), hipMemcpyDeviceToHost, ctx->stream));
  RV_TRY(hipStreamSynchronize(ctx->stream));
  if ((int)ctx->depth.size() < ctx->cfg.max_seq) ctx->depth.assign(ctx->cfg.max_seq, ctx->cfg.n_layers);
  for (int p = first; p <= last; ++p) ctx->depth[p] = E;
  for (int p = first - 1; p >= 0 && ctx->depth[p] < E; --p) ctx->depth[p] = E;
  return RIVER_OK;
}

void drop_graphs(river_ctx *ctx) {
  for (auto &kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  ctx->graphs.clear();
}

void drop_events(river_ctx *ctx) {
  for (auto &t : ctx->timed) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  ctx->timed.clear();
  for (auto e : ctx->event_pool) (void)hipEventDestroy(e);
  ctx->event_pool.clear();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of river_debug_linear_noalloc: the batched-row GEMM's split-K partial
// tiles live in this file-scope device array instead of the context's
// workspace, so that entry point allocates nothing and needs no workspace
// room.  Every GPU the library runs on holds its own copy (32 MiB) until the
// process ends; host code uses only the device address hipGetSymbolAddress
// returns for it on that device (the array's name is a host-side stand-in).
// Every call on one GPU shares that GPU's copy: calls that overlap on one GPU
// race.  Each call writes every partial tile it later reads, so nothing needs
// clearing between calls.
// ---------------------------------------------------------------------------
static constexpr int64_t kScratchFloats = int64_t(8) << 20;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s (the current device
// for the null stream), resolved once per device with that device current.
int scratch_for_stream(hipStream_t s, float **out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return RIVER_E_HIP;
  dev = cur;
  if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return RIVER_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RIVER_E_UNIMPLEMENTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return RIVER_E_HIP;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return RIVER_E_HIP;
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  *out = g_scratch_ptr[dev];
  return RIVER_OK;
}

int debug_linear(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit, const void *d_x,
                 int32_t M, float *d_y, float *part, int64_t part_cap);

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *river_strerror(int code) {
  switch (code) {
    case RIVER_OK: return "ok";
    case RIVER_E_INVALID_ARG: return "invalid argument";
    case RIVER_E_BAD_SIZE: return "buffer smaller than required";
    case RIVER_E_STATE: return "call out of order";
    case RIVER_E_RANGE: return "batch or position out of range";
    case RIVER_E_HIP: return "HIP runtime error";
    case RIVER_E_UNIMPLEMENTED: return "shape not supported by the kernels";
  }
  return "unknown status";
}

int river_query_sizes(const river_config *cfg, river_sizes *out) {
  if (!cfg || !out) return RIVER_E_INVALID_ARG;
  if (!valid_config(cfg)) return RIVER_E_INVALID_ARG;
  const int sup = supported(cfg);
  if (sup != RIVER_OK) return sup;
  out->exit_bank_bytes = bank_bytes(*cfg, false);
  out->exit_bank_copy_bytes = bank_bytes(*cfg, true);
  out->kv_cache_bytes = (size_t)2 * cfg->n_layers * cfg->max_batch * cfg->n_kv_heads *
                        cfg->max_seq * cfg->head_dim * 2;
  out->workspace_bytes = workspace_layout(*cfg).total;
  out->control_bytes = control_bytes(cfg->max_batch, cfg->n_kv_heads, cfg->max_seq);
  return RIVER_OK;
}

int river_exit_bank_offsets(const river_config *cfg, int32_t layer, int32_t linear,
                            int32_t copy_layout, size_t *codes_off, size_t *sz_off) {
  if (!cfg || !codes_off || !sz_off || !valid_config(cfg)) return RIVER_E_INVALID_ARG;
  if (layer < 0 || layer >= cfg->n_layers || linear < 0 || linear >= 7) return RIVER_E_RANGE;
  const int sup = supported(cfg);
  if (sup != RIVER_OK) return sup;
  bank_offsets(*cfg, layer, linear, copy_layout != 0, codes_off, sz_off);
  return RIVER_OK;
}

int river_init(const river_config *cfg, const river_weights *w, void *exit_bank, void *kv_cache,
               void *workspace, void *control, const river_sizes *given, void *hip_stream,
               river_ctx **out) {
  if (!cfg || !w || !exit_bank || !kv_cache || !workspace || !control || !given || !out)
    return RIVER_E_INVALID_ARG;
  if (!valid_config(cfg)) return RIVER_E_INVALID_ARG;
  river_sizes need;
  const int q = river_query_sizes(cfg, &need);
  if (q != RIVER_OK) return q;
  if (given->exit_bank_bytes < need.exit_bank_bytes || given->kv_cache_bytes < need.kv_cache_bytes ||
      given->workspace_bytes < need.workspace_bytes || given->control_bytes < need.control_bytes)
    return RIVER_E_BAD_SIZE;
  if (!w->embed || !w->final_norm || !w->layers) return RIVER_E_INVALID_ARG;
  if (!cfg->tied_embeddings && !w->lm_head) return RIVER_E_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const river_layer_w &L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.w_gate || !L.w_up ||
        !L.w_down)
      return RIVER_E_INVALID_ARG;
  }
  river_ctx *ctx = new (std::nothrow) river_ctx();
  if (!ctx) return RIVER_E_INVALID_ARG;
  ctx->cfg = *cfg;
  ctx->layers.assign(w->layers, w->layers + cfg->n_layers);
  ctx->embed = static_cast<const uint16_t *>(w->embed);
  ctx->final_norm = static_cast<const uint16_t *>(w->final_norm);
  ctx->lm_head = static_cast<const uint16_t *>(cfg->tied_embeddings ? w->embed : w->lm_head);
  ctx->bank = static_cast<char *>(exit_bank);
  ctx->bank_size = given->exit_bank_bytes;
  ctx->kv = static_cast<uint16_t *>(kv_cache);
  ctx->ws = static_cast<char *>(workspace);
  ctx->ctrl = static_cast<Control *>(control);
  ctx->stream = static_cast<hipStream_t>(hip_stream);
  ctx->wl = workspace_layout(*cfg);
  *out = ctx;
  return RIVER_OK;
}

int river_build_exit_layers(river_ctx *ctx, int32_t mode) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  if (mode != RIVER_EXIT_INT4 && mode != RIVER_EXIT_COPY && mode != RIVER_EXIT_HQQ)
    return RIVER_E_INVALID_ARG;
  const bool copy = mode == RIVER_EXIT_COPY;
  if (ctx->bank_size < bank_bytes(ctx->cfg, copy)) return RIVER_E_BAD_SIZE;
  const river_config &c = ctx->cfg;
  drop_graphs(ctx);
  ctx->built = false;
  RV_TRY(launch_clear(ctx->ctrl, control_bytes(c.max_batch, c.n_kv_heads, c.max_seq), ctx->stream));
  ctx->ctrl_tau_bits = 0;   // the cleared block holds tau = +0.0
  RV_TRY(launch_rope_table(at<float2>(ctx->ws, ctx->wl.rope), c.max_seq, c.head_dim, c.rope_theta,
                           ctx->stream));
  LinearShape sh[7];
  linear_shapes(c, sh);
  // offloaded backbone layers: their linears live in host memory
  ctx->remote.assign(c.n_layers, 0);
  for (int l = 0; l < c.n_layers; ++l) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, ctx->layers[l].wq) == hipSuccess && a.type == hipMemoryTypeHost)
      ctx->remote[l] = 1;
  }
  (void)hipGetLastError();   // a pointer HIP does not know leaves an error behind
  for (int l = 0; l < c.n_layers; ++l) {
    const river_layer_w &L = ctx->layers[l];
    const void *src[7] = {L.wq, L.wk, L.wv, L.wo, L.w_gate, L.w_up, L.w_down};
    for (int i = 0; i < 7; ++i) {
      size_t co, so;
      bank_offsets(c, l, i, copy, &co, &so);
      if (copy) {
        // (hipMemcpyDefault: an offloaded backbone layer lives in host memory)
        RV_TRY(hipMemcpyAsync(ctx->bank + co, src[i], (size_t)sh[i].N * sh[i].K * 2,
                              hipMemcpyDefault, ctx->stream));
      } else if (mode == RIVER_EXIT_HQQ) {
        RV_TRY(launch_quantize_hqq(static_cast<const uint16_t *>(src[i]), sh[i].N, sh[i].K,
                                   c.group_size, at<uint32_t>(ctx->bank, co), at<uint32_t>(ctx->bank, so),
                                   kHqqIters, kHqqBeta, kHqqKappa, ctx->stream));
      } else {
        RV_TRY(launch_quantize(static_cast<const uint16_t *>(src[i]), sh[i].N, sh[i].K,
                               c.group_size, at<uint32_t>(ctx->bank, co), at<uint32_t>(ctx->bank, so),
                               ctx->stream));
      }
    }
  }
  ctx->built = true;
  // (the kernels see the bank's form: an HQQ-refined bank is an int4 bank)
  ctx->exit_mode = copy ? RIVER_EXIT_COPY : RIVER_EXIT_INT4;
  ctx->pos = 0;
  ctx->batch = 0;
  return RIVER_OK;
}

int river_prefill(river_ctx *ctx, const int32_t *d_tokens, int32_t B, int32_t T, float tau,
                  float *d_logits, int32_t *d_next) {
  if (!ctx || !d_tokens) return RIVER_E_INVALID_ARG;
  if (!std::isfinite(tau)) return RIVER_E_INVALID_ARG;
  if (!ctx->built) return RIVER_E_STATE;
  if (B < 1 || T < 1 || B > ctx->cfg.max_batch || T > ctx->cfg.max_seq) return RIVER_E_RANGE;
  if (ctx->rec && record_layout(ctx->cfg, (int64_t)B * T).total > ctx->rec_bytes)
    return RIVER_E_BAD_SIZE;
  if (ctx->strategy == kStratRecompute && B != 1) return RIVER_E_UNIMPLEMENTED;
  if (ctx->strategy == kStratRecompute && !ctx->kv_state) return RIVER_E_STATE;
  const int st = enqueue_prefill(ctx, d_tokens, B, T, tau, d_logits, d_next);
  // its begin kernel wrote tau (after a failure the value is unknown: a bit
  // pattern no finite tau has makes the next decode step write it again)
  if (st == RIVER_OK)
    std::memcpy(&ctx->ctrl_tau_bits, &tau, 4);
  else
    ctx->ctrl_tau_bits = 0x7FC00001u;
  if (st != RIVER_OK) return st;
  ctx->pos = T;
  ctx->batch = B;
  if (ctx->strategy == kStratRecompute) {
    ctx->depth.assign(ctx->cfg.max_seq, ctx->cfg.n_layers);
    RV_TRY_RC(note_depth(ctx, 0, T - 1));
  }
  return RIVER_OK;
}

// n decode steps enqueued back to back: step i reads its tokens from d_tokens
// (i = 0) or from the next tokens of step i - 1, d_next + (i - 1) B, and writes
// its own to d_next + i B (d_next may be null only for n = 1)
static int decode_steps(river_ctx *ctx, int n, const int32_t *d_tokens, float tau, float *d_logits,
                        int32_t *d_next) {
  if (!ctx || !d_tokens || n < 1 || n > kMaxStepsPerCall || (n > 1 && !d_next)) return RIVER_E_INVALID_ARG;
  if (!std::isfinite(tau)) return RIVER_E_INVALID_ARG;
  if (!ctx->built || ctx->batch == 0) return RIVER_E_STATE;
  if (ctx->pos + n > ctx->cfg.max_seq) return RIVER_E_RANGE;
  if (ctx->rec && record_layout(ctx->cfg, ctx->batch).total > ctx->rec_bytes)
    return RIVER_E_BAD_SIZE;
  // the comparator strategies run on the decode kernels of up to 8 rows; the
  // kv mask on the matrix-core attention
  if (ctx->strategy != kStratRiver && ctx->batch > 8) return RIVER_E_UNIMPLEMENTED;
  if (ctx->strategy == kStratMask && ctx->attn_kind != 0) return RIVER_E_UNIMPLEMENTED;
  // the recompute comparator: one sequence, a state buffer, and a prefill
  // under the same strategy before its steps; the host sizes each step's
  // launches from the earlier steps' exits, so one step per call
  const bool recompute = ctx->strategy == kStratRecompute;
  if (recompute && (ctx->batch != 1 || n != 1)) return RIVER_E_UNIMPLEMENTED;
  if (recompute && (!ctx->kv_state || (int)ctx->depth.size() < ctx->cfg.max_seq)) return RIVER_E_STATE;
  // the step reads tau from the control block: write it when it changes
  uint32_t tau_bits;
  std::memcpy(&tau_bits, &tau, 4);
  if (tau_bits != ctx->ctrl_tau_bits) {
    RV_TRY(launch_set_tau(ctx->ctrl, tau, ctx->stream));
    ctx->ctrl_tau_bits = tau_bits;
  }
  const int B = ctx->batch;
  auto enqueue_all = [&]() -> int {
    for (int i = 0; i < n; ++i) {
      const int32_t *tok = i == 0 ? d_tokens : d_next + (int64_t)(i - 1) * B;
      int32_t *nx = d_next ? d_next + (int64_t)i * B : nullptr;
      const int st = enqueue_decode(ctx, tok, tau, d_logits, nx);
      if (st != RIVER_OK) return st;
    }
    return RIVER_OK;
  };
  // (recompute: the launches of a step depend on the exits of the earlier
  // passes, so its steps run eagerly)
  if (ctx->use_graph && !ctx->profiling && !ctx->rec && ctx->stream != nullptr && !recompute) {
    const river_ctx::GraphKey key{d_tokens, d_logits, d_next, B, ctx->force_E, n};
    auto it = ctx->graphs.find(key);
    if (it == ctx->graphs.end()) {
      // every new (tokens, logits, next, steps) key records a graph; callers
      // that reuse their buffers hit the cache, the others are bounded here
      if (ctx->graphs.size() >= kMaxGraphs) drop_graphs(ctx);
      hipGraph_t graph = nullptr;
      RV_TRY(hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeThreadLocal));
      const int st = enqueue_all();
      hipError_t e = hipStreamEndCapture(ctx->stream, &graph);
      hipGraphExec_t exec = nullptr;
      if (st == RIVER_OK && e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      if (graph) (void)hipGraphDestroy(graph);
      if (st != RIVER_OK) return st;
      if (e != hipSuccess) return RIVER_E_HIP;
      it = ctx->graphs.emplace(key, exec).first;
    }
    RV_TRY(hipGraphLaunch(it->second, ctx->stream));
  } else {
    const int st = enqueue_all();
    if (st != RIVER_OK) return st;
  }
  if (recompute) RV_TRY_RC(note_depth(ctx, ctx->pos, ctx->pos));
  ctx->pos += n;
  return RIVER_OK;
}

int river_decode_step(river_ctx *ctx, const int32_t *d_tokens, float tau, float *d_logits,
                      int32_t *d_next) {
  return decode_steps(ctx, 1, d_tokens, tau, d_logits, d_next);
}

int river_decode_steps(river_ctx *ctx, int32_t n_steps, const int32_t *d_tokens, float tau,
                       float *d_logits, int32_t *d_next) {
  return decode_steps(ctx, n_steps, d_tokens, tau, d_logits, d_next);
}

int river_exit_stats(river_ctx *ctx, river_exit_stats_t *out) {
  if (!ctx || !out) return RIVER_E_INVALID_ARG;
  if (!ctx->built) return RIVER_E_STATE;
  Control h;
  RV_TRY(hipMemcpyAsync(&h, ctx->ctrl, sizeof(Control), hipMemcpyDeviceToHost, ctx->stream));
  RV_TRY(hipStreamSynchronize(ctx->stream));
  std::memset(out, 0, sizeof(*out));
  const int L = ctx->cfg.n_layers;
  double sum = 0.0;
  for (int e = 0; e <= L; ++e) {
    out->decode_hist[e] = h.decode_hist[e];
    out->prefill_hist[e] = h.prefill_hist[e];
    sum += (double)e * (double)h.decode_hist[e];
  }
  out->n_decode_steps = h.n_decode;
  out->n_prefill = h.n_prefill;
  out->mean_exit_layer = h.n_decode ? sum / (double)h.n_decode : 0.0;
  out->last_E = h.last_E;
  out->pos = h.pos;
  out->token_errors = h.bad_token;
  for (int l = 0; l < RIVER_MAX_LAYERS; ++l) out->last_trace[l] = l < L ? h.trace[l] : NAN;
  return RIVER_OK;
}

int river_set_option(river_ctx *ctx, int32_t option, int64_t value) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  switch (option) {
    case RIVER_OPT_GRAPH:
      if (value != 0 && value != 1) return RIVER_E_INVALID_ARG;
      ctx->use_graph = value != 0;
      return RIVER_OK;
    case RIVER_OPT_FORCE_E:
      if (value < -1 || value > ctx->cfg.n_layers) return RIVER_E_RANGE;
      ctx->force_E = (int)value;
      return RIVER_OK;
    case RIVER_OPT_ATTN_CHUNK:
      if (value != 0 && (value < kAttnSub || value % kAttnSub ||
                         (ctx->cfg.max_seq + value - 1) / value > kMaxAttnSplits))
        return RIVER_E_INVALID_ARG;
      ctx->attn_chunk = (int)value;
      drop_graphs(ctx);
      return RIVER_OK;
    case RIVER_OPT_ATTN:
      if (value != 0 && value != 1) return RIVER_E_INVALID_ARG;
      ctx->attn_kind = (int)value;
      drop_graphs(ctx);
      return RIVER_OK;
    case RIVER_OPT_GEMV:
      if (value < 0 || value > 2) return RIVER_E_INVALID_ARG;
      ctx->gemv_mode = (int)value;
      drop_graphs(ctx);
      return RIVER_OK;
    case RIVER_OPT_KV_STRATEGY:
      if (value < kStratRiver || value > kStratRecompute) return RIVER_E_INVALID_ARG;
      ctx->strategy = (int)value;
      ctx->depth.clear();   // (a recompute sequence starts at its prefill)
      drop_graphs(ctx);
      return RIVER_OK;
    case RIVER_OPT_PROFILE:
      if (value != 0 && value != 1) return RIVER_E_INVALID_ARG;
      if (!value) drop_events(ctx);
      ctx->profiling = value != 0;
      return RIVER_OK;
  }
  return RIVER_E_INVALID_ARG;
}

int river_time_kernel(river_ctx *ctx, int32_t kind, int32_t reps, double *avg_us) {
  if (!ctx || !avg_us || reps < 1) return RIVER_E_INVALID_ARG;
  if (kind < RIVER_K_QKV || kind > RIVER_K_DOWN) return RIVER_E_INVALID_ARG;
  if (!ctx->built || ctx->batch == 0) return RIVER_E_STATE;
  if (ctx->stream == nullptr) return RIVER_E_STATE;
  char *rec = ctx->rec;
  const bool prof = ctx->profiling;
  ctx->rec = nullptr;
  ctx->profiling = false;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  int st = RIVER_OK;
  hipError_t e = hipStreamBeginCapture(ctx->stream, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    st = enqueue_decode(ctx, nullptr, 0.f, nullptr, nullptr, kind);
    e = hipStreamEndCapture(ctx->stream, &graph);
  }
  ctx->rec = rec;
  ctx->profiling = prof;
  if (st != RIVER_OK) return st;
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (graph) (void)hipGraphDestroy(graph);
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipGraphLaunch(exec, ctx->stream);   // warm-up replay
  if (e == hipSuccess) e = hipEventRecord(a, ctx->stream);
  for (int i = 0; i < reps && e == hipSuccess; ++i) e = hipGraphLaunch(exec, ctx->stream);
  if (e == hipSuccess) e = hipEventRecord(b, ctx->stream);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (e != hipSuccess) return RIVER_E_HIP;
  *avg_us = (double)ms * 1e3 / ((double)reps * ctx->cfg.n_layers);
  return RIVER_OK;
}

int river_record_bytes(const river_config *cfg, int32_t rows, size_t *bytes) {
  if (!cfg || !bytes || !valid_config(cfg) || rows < 1) return RIVER_E_INVALID_ARG;
  *bytes = record_layout(*cfg, rows).total;
  return RIVER_OK;
}

int river_set_record(river_ctx *ctx, void *d_buf, size_t bytes) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  if (d_buf && bytes < record_layout(ctx->cfg, 1).total) return RIVER_E_BAD_SIZE;
  ctx->rec = static_cast<char *>(d_buf);
  ctx->rec_bytes = d_buf ? bytes : 0;
  return RIVER_OK;
}

int river_set_kv_state(river_ctx *ctx, void *d_buf, size_t bytes) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  if (d_buf && (bytes < (size_t)ctx->cfg.max_seq * ctx->cfg.d_model * 4 ||
                reinterpret_cast<uintptr_t>(d_buf) % 16))
    return RIVER_E_BAD_SIZE;
  ctx->kv_state = static_cast<float *>(d_buf);
  ctx->depth.clear();
  return RIVER_OK;
}

int river_reset(river_ctx *ctx) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  ctx->pos = 0;
  ctx->batch = 0;
  ctx->depth.clear();
  return RIVER_OK;
}

int river_profile_read(river_ctx *ctx, river_kernel_time_t *out) {
  if (!ctx || !out) return RIVER_E_INVALID_ARG;
  if (!ctx->profiling) return RIVER_E_STATE;
  RV_TRY(hipStreamSynchronize(ctx->stream));
  for (int k = 0; k < RIVER_K_NKINDS; ++k) out[k] = {0, 0.0};
  for (auto &t : ctx->timed) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess && t.kind >= 0 && t.kind < RIVER_K_NKINDS) {
      out[t.kind].launches += 1;
      out[t.kind].total_ms += ms;
    }
    ctx->event_pool.push_back(t.a);
    ctx->event_pool.push_back(t.b);
  }
  ctx->timed.clear();
  return RIVER_OK;
}

int river_debug_linear(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit,
                       const void *d_x, int32_t M, float *d_y) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  return debug_linear(ctx, layer, linear, use_exit, d_x, M, d_y, at<float>(ctx->ws, ctx->wl.mg_part),
                      ctx->wl.mg_part_floats);
}

int river_debug_linear_noalloc(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit,
                               const void *d_x, int32_t M, float *d_y) {
  if (!ctx) return RIVER_E_INVALID_ARG;
  float *part = nullptr;
  const int st = scratch_for_stream(ctx->stream, &part);
  if (st != RIVER_OK) return st;
  return debug_linear(ctx, layer, linear, use_exit, d_x, M, d_y, part, kScratchFloats);
}

}  // extern "C"

namespace {

// One linear through the production cores; the batched-row GEMM's split-K
// partial tiles go to `part` (capacity part_cap floats).
int debug_linear(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit, const void *d_x,
                 int32_t M, float *d_y, float *part, int64_t part_cap) {
  if (!ctx || !d_x || !d_y) return RIVER_E_INVALID_ARG;
  if (!ctx->built) return RIVER_E_STATE;
  const river_config &c = ctx->cfg;
  if (layer < 0 || layer >= c.n_layers || linear < 0 || linear >= 7 || M < 1 ||
      (use_exit != 0 && use_exit != 1))
    return RIVER_E_RANGE;
  LinearShape sh[7];
  linear_shapes(c, sh);
  const int path = use_exit ? kPathExit : kPathBackbone;
  if (M <= 8) {
    GemvParams g{};
    fill_weights(ctx, layer, linear, 1, g.w);
    g.N = sh[linear].N; g.K = sh[linear].K; g.G = c.group_size;
    g.gemv_mode = ctx->gemv_mode;
    g.gshift = __builtin_ctz((unsigned)c.group_size);
    g.layer = layer; g.exit_mode = ctx->exit_mode; g.ctrl = ctx->ctrl; g.B = M;
    g.x_src = static_cast<const uint16_t *>(d_x); g.x_stride = sh[linear].K;
    g.path = path; g.y_out = d_y; g.y_stride = sh[linear].N;
    RV_TRY(launch_gemv(kXBf16, kEpPlain, g, ctx->stream));
  } else {
    GemmParams g = mgemm_base(ctx, layer, M);
    fill_weights(ctx, layer, linear, 1, g.w);
    g.M = M; g.N = sh[linear].N; g.K = sh[linear].K;
    g.x = static_cast<const uint16_t *>(d_x); g.ldx = sh[linear].K;
    g.path = path; g.y_out = d_y; g.y_stride = sh[linear].N;
    if (M <= 64 && ctx->cfg.max_batch > 8) {
      // the decode core of 9..64 rows
      g.part = part;
      g.part_cap = part_cap;
      if (mgemm_part_floats_max(M, sh[linear].N, sh[linear].K) > part_cap) return RIVER_E_BAD_SIZE;
      RV_TRY(launch_mgemm(kEpPlain, g, ctx->stream));
    } else {
      RV_TRY(launch_prefill_gemm(kEpPlain, g, ctx->stream));   // the prefill core
    }
  }
  return RIVER_OK;
}

}  // namespace

extern "C" {

void river_destroy(river_ctx *ctx) {
  if (!ctx) return;
  drop_graphs(ctx);
  drop_events(ctx);
  delete ctx;
}

}  // extern "C"
