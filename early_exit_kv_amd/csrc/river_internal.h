// Internal declarations shared by the host scheduler and the HIP kernels of
// the KV-shared early-exit decoder.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "river.h"

namespace river {

// ---------------------------------------------------------------------------
// Device control block.  It lives at the start of the caller's control buffer
// and carries everything a pass decides on the device: the sticky exit flag,
// the number of backbone layers run, tau, the cache position, the per-layer
// trace of batch-minimum cosines, histograms of E, and the counters of the
// "last workgroup finishes the reduction" pattern.  Counters are zero between
// kernels: the workgroup that finds itself last resets its counter.
// ---------------------------------------------------------------------------
constexpr int kMaxLayers = RIVER_MAX_LAYERS;
constexpr int kNumCounters = 16;

enum CounterId {
  kCtrExit = 0,       // decode down-projection: exit test after the layer
  kCtrLogits = 1,     // LM head: argmax hand-off and bookkeeping
  kCtrRowsCos = 2,    // prefill: cosine minimum over all rows
};

struct Control {
  int32_t flag;      // 1 once the exit fired in the current pass
  int32_t E;         // backbone layers run in the current pass
  float tau;
  int32_t pos;       // position the current decode step writes
  int32_t force_E;   // -1: decide with tau; e >= 0: layers >= e are exit layers
  int32_t bad_token; // a token id outside [0, vocab) was seen (and clamped)
  int32_t last_E;
  int32_t strategy;  // KvStrategy of the current pass
  int64_t n_decode, n_prefill;
  int64_t decode_hist[kMaxLayers + 1];
  int64_t prefill_hist[kMaxLayers + 1];
  float trace[kMaxLayers];
  uint32_t counters[kNumCounters];
  // followed by: uint64_t argmax_key[max_batch];
  //              uint32_t attn_counters[max_batch * n_kv_heads];
  //              int32_t pos_E[max_seq]  (E of the pass that wrote each position)
};

// What the layers at and past the exit do (RIVER_OPT_KV_STRATEGY): run as
// exit layers (the method), or, as comparators, four prior fixes of the
// missing K/V of early-exited tokens: skipped with later tokens leaving out
// the K/V that are missing (kv mask), only their K/V computed from the exit
// state (state propagation), skipped with the exit layer never increasing
// along the sequence (mono-decreasing), skipped with the missing K/V computed
// when a later pass reaches the layer (batching recompute).
enum KvStrategy { kStratRiver = 0, kStratMask = 1, kStratPropagate = 2, kStratMono = 3, kStratRecompute = 4 };

__host__ __device__ inline size_t control_bytes(int max_batch, int n_kv_heads, int max_seq) {
  size_t b = sizeof(Control);
  b = (b + 7) & ~size_t(7);
  b += sizeof(uint64_t) * (size_t)max_batch;
  b += sizeof(uint32_t) * (size_t)max_batch * n_kv_heads;
  b += sizeof(int32_t) * (size_t)max_seq;
  return (b + 255) & ~size_t(255);
}
__host__ __device__ inline uint64_t *control_keys(Control *c) {
  size_t off = (sizeof(Control) + 7) & ~size_t(7);
  return reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(c) + off);
}
__host__ __device__ inline uint32_t *control_attn_counters(Control *c, int max_batch) {
  return reinterpret_cast<uint32_t *>(control_keys(c) + max_batch);
}
__host__ __device__ inline int32_t *control_pos_E(Control *c, int max_batch, int n_kv_heads) {
  return reinterpret_cast<int32_t *>(control_attn_counters(c, max_batch) + (size_t)max_batch * n_kv_heads);
}

// ---------------------------------------------------------------------------
// Exit-bank layout: per layer, per linear (q, k, v, o, gate, up, down), the
// packed codes then the packed scale/zero words, each region 256-byte aligned.
// ---------------------------------------------------------------------------
struct LinearShape {
  int N, K;
};
void linear_shapes(const river_config &c, LinearShape out[7]);
size_t align256(size_t x);
// offsets of (layer, linear) in the int4 bank or in the bf16 copy bank
void bank_offsets(const river_config &c, int layer, int linear, bool copy, size_t *codes,
                  size_t *sz);
size_t bank_bytes(const river_config &c, bool copy);

// ---------------------------------------------------------------------------
// Workspace layout (byte offsets into the caller's workspace buffer).
// ---------------------------------------------------------------------------
struct Workspace {
  size_t hA, hB;       // fp32 residual stream [R][d], layer input / output
  size_t x;            // bf16 normalised activations [R][max(d, F)] (prefill)
  size_t q;            // bf16 queries [R][Hq*Dh]
  size_t attn;         // bf16 attention output [R][Hq*Dh]
  size_t u;            // bf16 SwiGLU product [R][F]
  size_t part;         // fp32 per-workgroup partial sums for the exit test
  size_t attn_part;    // fp32 split-K attention partials
  size_t rope;         // fp32 (cos, sin) of pos * theta^(-2i/Dh), [max_seq][Dh/2]
  size_t mg_part;      // fp32 split-K partials of the batched-row GEMM
  size_t pg_part;      // fp32 split-K partials of the prefill GEMM (o, down; up to 512 rows)
  size_t total;
  int64_t rows;        // R: rows the buffers hold
  int part_floats;
  int attn_splits;     // split count the decode attention is sized for
  int64_t mg_part_floats;
  int64_t pg_part_floats;
};
Workspace workspace_layout(const river_config &c);

constexpr int kAttnSub = 64;      // positions per decode-attention sub-chunk
constexpr int kMaxAttnSplits = 512;  // splits one (b, kv head) may use
constexpr int kPartFloatsPerWG = 3 * 64;  // B <= 64 rows x (dot, |a|^2, |b|^2)

// ---------------------------------------------------------------------------
// Kernel launch parameters
// ---------------------------------------------------------------------------
enum XSource { kXNorm = 0, kXBf16 = 1 };
enum Epilogue { kEpQKV = 0, kEpResid = 1, kEpResidExit = 2, kEpSwiGLU = 3, kEpLogits = 4, kEpPlain = 5 };
// weight path of a launch: decided on the device, or fixed (debug entry point,
// forced exit).  kPathPending (the recompute comparator's rows of earlier
// positions): backbone weights, and the launch does nothing once the current
// pass is past its exit at this layer.
enum PathChoice { kPathDevice = 0, kPathBackbone = 1, kPathExit = 2, kPathPending = 3 };

struct LinearWeights {
  const uint16_t *bf[3];   // backbone bf16 segments (or exit bf16 copies)
  const uint32_t *q4[3];   // exit int4 code segments
  const uint32_t *sz[3];   // exit scale/zero segments
  const uint16_t *ex_bf[3];// exit bf16 copy segments (copy mode)
  int seg_rows[3];         // physical rows of each segment
  int nseg;
};

struct GemvParams {
  LinearWeights w;
  int N;            // logical output rows
  int K;            // input columns
  int G;            // group size
  int layer;        // layer index (exit choice); -1: always backbone (LM head)
  int exit_mode;    // RIVER_EXIT_INT4 or RIVER_EXIT_COPY
  Control *ctrl;
  int B;            // batch rows
  // x source
  const float *h_src; int64_t h_stride;   // kXNorm: fp32 rows, stride in floats
  const uint16_t *gain; float eps;
  const uint16_t *x_src; int64_t x_stride; // kXBf16
  // epilogues
  const float *h_in; float *h_out; int64_t h_io_stride;   // residual
  // (kEpResidExit also reads the layer input through h_src, same stride)
  uint16_t *q_out; uint16_t *k_cache; uint16_t *v_cache;  // QKV
  int Hq, Hkv, Dh, max_seq, max_batch; float rope_theta;
  const float2 *rope;                                     // (cos, sin) table
  uint16_t *u_out; int64_t u_stride;                      // SwiGLU
  float *part;                                            // exit test partials
  int test_exit; int n_layers;                            // down: write the partials
  int test_prev; int part_wgs;    // QKV: decide the previous layer's test first
  int gshift;                     // log2(group size)
  int path;                       // PathChoice
  float *y_out; int64_t y_stride; // kEpPlain: fp32 [B][N]
  float *logits; int32_t *next; int is_prefill; int vocab;// LM head
  int gemv_mode;                  // 0 per-linear choice, 1 dot-product GEMV, 2 MFMA GEMV where it fits
  int remote_bb;                  // the backbone weights live in host memory: while the exit
                                  // test is pending, stream the exit copy first
};


struct AttnParams {
  const uint16_t *q;      // [B][Hq*Dh]
  const uint16_t *k_cache, *v_cache;  // layer base: [max_batch][Hkv][S][Dh]
  uint16_t *out;          // [B][Hq*Dh]
  float *part;            // [B][Hq][splits][Dh + 2]
  uint32_t *counters;     // [B][Hkv]
  Control *ctrl;
  int B, Hq, Hkv, Dh, S, splits, chunk;
  float scale;
  int mfma;               // 1: scores on the matrix cores
  int layer;              // the layer (kernels past the exit return at once in the comparators)
  const int32_t *pos_E;   // kv mask: E per earlier position (positions whose E <= layer
                          // hold no K/V here); nullptr: every position
  int nw8;                // matrix-core kernel with eight wavefronts (one split, chunk a multiple of 128)
};
// positions per decode-attention workgroup for a cache of max_seq positions
int attn_chunk(int max_seq, int batch, int n_kv_heads);

struct BeginParams {
  Control *ctrl;
  const int32_t *tokens;
  int64_t rows;       // tokens to embed
  int B;              // batch rows (argmax keys to clear)
  const uint16_t *embed;
  float *h;
  int d, vocab, n_layers, force_E;
  float tau;
  int write_tau;      // 1: write tau into the control block (prefill); decode
                      // steps read the tau launch_set_tau left there, so one
                      // recorded step serves every tau
  int is_prefill;
  int set_pos;        // >= 0: write this position into the control block
  int strategy;       // KvStrategy of the pass
};

// ---- launchers (each returns hipGetLastError() after the launch) ----------
// Launch with an argument array (one place for every pass kernel).
hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds,
                         hipStream_t s);
template <typename P>
hipError_t launch_1(void (*kernel)(P), dim3 grid, dim3 block, const P &p, hipStream_t s) {
  P copy = p;
  void *args[] = {&copy};
  return launch_kernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, s);
}

hipError_t launch_clear(void *p, size_t bytes, hipStream_t s);
hipError_t launch_quantize(const uint16_t *w, int N, int K, int G, uint32_t *codes, uint32_t *sz,
                           hipStream_t s);
// the min-max quantiser followed by `iters` HQQ-style rounds on the zero point
hipError_t launch_quantize_hqq(const uint16_t *w, int N, int K, int G, uint32_t *codes, uint32_t *sz,
                               int iters, float beta, float kappa, hipStream_t s);
// defaults of those rounds (the half-quadratic solver's published settings)
constexpr int kHqqIters = 20;
constexpr float kHqqBeta = 10.0f;
constexpr float kHqqKappa = 1.01f;
hipError_t launch_begin(const BeginParams &p, hipStream_t s);
// one thread writes tau into the control block
hipError_t launch_set_tau(Control *c, float tau, hipStream_t s);
// after a pass (kv mask): pos_E of the positions it wrote = its E (n > 0: the
// first n positions, a prefill; n = 0: position pos - 1, a decode step)
hipError_t launch_set_pos_E(Control *c, int32_t *pos_E, int n, hipStream_t s);
// RoPE table: rope[t][i] = (cos, sin)(t * theta^(-2i/Dh)), angles in float64
hipError_t launch_rope_table(float2 *rope, int max_seq, int head_dim, float theta, hipStream_t s);
hipError_t launch_gemv(XSource xs, Epilogue ep, const GemvParams &p, hipStream_t s);
// workgroups launch_gemv uses for these parameters (the QKV launch reads that
// many partials left by the previous layer's down projection)
int gemv_grid(Epilogue ep, const GemvParams &p);
// the matrix-core GEMV handles these parameters (LDS, group size, K)
bool mgemv_fits(Epilogue ep, const GemvParams &p);
hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s);

// prefill
struct RowsNormParams {
  const float *h; uint16_t *x; const uint16_t *gain; int64_t rows; int d; float eps;
  int64_t h_stride;   // floats between input rows (0: d)
  const Control *ctrl; int layer; int path;   // ctrl set: nothing where the layer is skipped past the exit
};
hipError_t launch_rows_norm(const RowsNormParams &p, hipStream_t s);
// dst[i] = src[i] for i < n, unless the current pass is past its exit at
// `layer` (the path's rule; the recompute comparator's state write-back)
hipError_t launch_rows_copy_run(float *dst, const float *src, int64_t n, const Control *ctrl, int layer,
                                int path, hipStream_t s);

struct GemmParams {
  LinearWeights w;
  int M, N, K, G;
  int layer, exit_mode;
  Control *ctrl;
  const uint16_t *x; int64_t ldx;  // bf16 [M][K]
  // epilogues (same meaning as GemvParams)
  const float *h_in; float *h_out; int64_t h_io_stride;
  uint16_t *q_out; uint16_t *k_cache; uint16_t *v_cache;
  int Hq, Hkv, Dh, max_seq, max_batch, T; float rope_theta;
  int start;                       // T > 0: row t of a sequence sits at position start + t
  const float2 *rope;
  uint16_t *u_out;
  int path;                        // PathChoice
  float *y_out; int64_t y_stride;  // kEpPlain
  // batched-row GEMM (mgemm) only
  float *logits; int32_t *next; int vocab; int is_prefill;   // kEpLogits
  float *part;                                               // split-K partial tiles
  int64_t part_cap;                                          // floats at part
  int nsplit, ks;                                            // K splits, K per split
  int ring;                                                  // int4 ring column block, 0: none (set at launch)
};

// Batched-row GEMM for 9..64 rows (decode of larger batches, LM head of
// prefill): weights stream from HBM straight into MFMA operands, the rows sit
// in LDS.  Plan: 16-row blocks, 128-column workgroups, K split over nsplit
// workgroups whose partial tiles a second kernel adds up.
constexpr int kMgemmBN = 128;
struct MgemmPlan { int mb, ncolblk, nsplit, ks, rbn; };   // rbn: int4 ring column block (0: none)
MgemmPlan mgemm_plan(int M, int ncols, int K);
int64_t mgemm_part_floats(const MgemmPlan &pl);
// split-K partial floats the launch of a linear of ncols x K at M rows may
// need (either plan)
int64_t mgemm_part_floats_max(int M, int ncols, int K);
hipError_t launch_mgemm(Epilogue ep, const GemmParams &p, hipStream_t s);
hipError_t launch_gemm(Epilogue ep, const GemmParams &p, hipStream_t s);
// Prefill GEMM for many rows (128 x 128 tiles; shapes where pgemm_fits holds).
bool pgemm_fits(int K, int G);
hipError_t launch_pgemm(Epilogue ep, const GemmParams &p, hipStream_t s);

struct AttnPrefillParams {
  const uint16_t *q;       // [B*T][Hq*Dh]
  const uint16_t *k_cache, *v_cache;  // layer base [max_batch][Hkv][S][Dh]
  uint16_t *out;           // [B*T][Hq*Dh]
  int B, T, Hq, Hkv, Dh, S;
  float scale;
  int mfma;                // 1: the matrix-core (flash-style) kernel, 0: the vector-ALU one
  Control *ctrl; int layer; int path;   // past the exit in the comparators: return at once
  int start;               // query row t sits at position start + t and sees keys 0 .. start + t
};
hipError_t launch_attn_prefill(const AttnPrefillParams &p, hipStream_t s);

struct RowsCosParams {
  const float *a, *b; int64_t rows; int d;
  float *part; Control *ctrl; int layer; int n_layers;
};
hipError_t launch_rows_cos_exit(const RowsCosParams &p, hipStream_t s);
// Exit test of a layer of many rows and the RMSNorm of its output rows for the
// next layer, one launch (n.h must be c.b, unit row stride).
hipError_t launch_rows_cos_norm(const RowsCosParams &c, const RowsNormParams &n, bool test, hipStream_t s);

}  // namespace river
