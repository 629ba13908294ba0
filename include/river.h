/*
 * river.h -- C ABI of the KV-shared early-exit decoder for MI355X (gfx950).
 *
 * The method is the one of the page "River-LLM: Large Language Model Seamless
 * Exit Based on KV Share" (arXiv:2604.18396):
 *   - section 3: beside every decoder layer sits an exit layer, a full copy of
 *     the layer's parameters quantised to 4-bit weights with 16-bit activations
 *     (W4A16), built without training; exit layers write their K/V into the
 *     cache slot of the original layer, so there is a single shared KV cache
 *     and later tokens never miss an entry;
 *   - section 4: after a layer, the state-transition similarity (cosine
 *     between the layer's input and output residual stream) is taken for every
 *     token of the batch; if its minimum exceeds tau, all remaining layers run
 *     as exit layers and no deeper layer tests again;
 *   - section 5: prefill takes one sequence-level decision for all prompt
 *     tokens, generation one decision per generated position.
 *
 * Conventions shared by every entry point
 *   - Every device buffer is allocated by the caller and only borrowed by the
 *     library; it must stay alive until river_destroy().  The library owns only
 *     its host-side context (and the HIP graphs it records for decode steps).
 *   - All GPU work is enqueued on the HIP stream given to river_init(); no call
 *     synchronises except river_exit_stats().  A kernel fault surfaces at the
 *     next synchronisation, as usual for HIP.
 *   - Every call returns a river status code.  Arguments and state are checked
 *     on the host before anything is enqueued: a call rejected by those checks
 *     enqueues nothing and leaves the context unchanged.  A HIP error met
 *     while enqueueing (RIVER_E_HIP) can leave the launches made before it on
 *     the stream; the pass is then incomplete and should be repeated from a
 *     prefill.  No C++ exception crosses the ABI.
 *   - bf16 means bfloat16 stored as 16-bit words; matrices are row-major
 *     [rows][cols], a linear layer's weight is [out N][in K] (y = x W^T).
 *   - The context is not thread-safe: calls on one context must not overlap.
 */
#ifndef RIVER_H
#define RIVER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct river_ctx river_ctx; /* opaque, owned by the library */

/* ---- status codes ------------------------------------------------------ */
enum {
  RIVER_OK = 0,
  RIVER_E_INVALID_ARG = 1,   /* null pointer, bad enum, non-finite tau, ...   */
  RIVER_E_BAD_SIZE = 2,      /* a buffer smaller than river_query_sizes says  */
  RIVER_E_STATE = 3,         /* call out of order (e.g. prefill before build) */
  RIVER_E_RANGE = 4,         /* batch > max_batch, position beyond max_seq    */
  RIVER_E_HIP = 5,           /* a HIP runtime call or kernel launch failed    */
  RIVER_E_UNIMPLEMENTED = 6  /* a shape the kernels do not support            */
};

/* ---- exit-bank construction modes -------------------------------------- */
enum {
  RIVER_EXIT_INT4 = 1, /* copy + 4-bit group quantisation (the method)         */
  RIVER_EXIT_COPY = 2, /* exact bf16 copy: exit layers equal the backbone; used
                          to check that the exit plumbing changes nothing      */
  RIVER_EXIT_HQQ = 3   /* RIVER_EXIT_INT4 followed by an HQQ-style refinement
                          of every group's zero point (same bank layout)       */
};

#define RIVER_MAX_LAYERS 256

/* Decoder shape (Llama-style: pre-norm RMSNorm, GQA attention with rotate-half
 * RoPE, SwiGLU MLP) and the capacity of the shared KV cache.
 *   head_dim must be even and at most 128; d_model, head_dim, ffn_dim multiples
 *   of 8; group_size a multiple of 32 dividing d_model, ffn_dim and
 *   n_q_heads*head_dim; n_q_heads a multiple of n_kv_heads. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps, rope_theta;
  int32_t tied_embeddings; /* 1: the LM head is the embedding matrix          */
  int32_t group_size;      /* G: input columns sharing one scale/zero          */
  int32_t max_batch;       /* rows of one decode step (and prefill batch)      */
  int32_t max_seq;         /* positions the shared cache holds per row         */
} river_config;

/* One decoder layer's backbone weights, pointers to bf16 that the device can
 * read:
 *   attn_norm, mlp_norm [d_model]; wq [Hq*Dh][d]; wk, wv [Hkv*Dh][d];
 *   wo [d][Hq*Dh]; w_gate, w_up [F][d]; w_down [d][F].
 * Backbone offloading (lead page, section 5: deep backbone layers leave
 * device memory, the exit layers stay): the seven linear matrices of a layer
 * may live in pinned host memory mapped into the device's address space
 * (hipHostMalloc, or a pinned allocation made by the caller's framework; pass
 * the device-side address hipHostGetDevicePointer gives).  The kernels then
 * read them over the host link, and only when the device-side decision runs
 * that layer on its backbone: once the exit has fired, the step reads the
 * int4 exit copy in HBM instead.  The exit bank, the norm gains, the
 * embedding, the LM head and the KV cache stay in device memory.  The first
 * kernel after a pending exit test starts streaming the backbone weights
 * before the test is decided, so an offloaded layer right after a tested one
 * is touched (a few KB) even when the exit fires. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} river_layer_w;

/* Whole-model weights: embed [V][d] bf16, final_norm [d] bf16, lm_head [V][d]
 * bf16 (NULL when tied_embeddings), layers: HOST array of n_layers entries
 * (copied by river_init, so it may be freed afterwards). */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const river_layer_w *layers;
} river_weights;

/* Device-buffer sizes in bytes, from river_query_sizes(). */
typedef struct {
  size_t exit_bank_bytes; /* packed int4 exit layers (river_exit_bank_offsets)    */
  size_t exit_bank_copy_bytes; /* bank size RIVER_EXIT_COPY needs (bf16 copies)    */
  size_t kv_cache_bytes;  /* the single shared cache, see below                    */
  size_t workspace_bytes; /* activations and reduction scratch                     */
  size_t control_bytes;   /* decision flag, tau, position, histograms, trace       */
} river_sizes;

/* Statistics read back by river_exit_stats().  E is the number of backbone
 * layers a pass ran (1..n_layers; n_layers means no exit). */
typedef struct {
  int64_t prefill_hist[RIVER_MAX_LAYERS + 1]; /* count of prefills per E        */
  int64_t decode_hist[RIVER_MAX_LAYERS + 1];  /* count of decode steps per E    */
  int64_t n_prefill, n_decode_steps;
  double mean_exit_layer;                     /* mean E over decode steps       */
  int32_t last_E;                             /* E of the latest pass           */
  int32_t pos;                                /* next position to be written    */
  int32_t token_errors;                       /* 1 if a token id outside
                                                 [0, vocab) was seen; it was
                                                 replaced by 0                  */
  float last_trace[RIVER_MAX_LAYERS];         /* latest pass: batch-min cosine
                                                 after layer l, NaN if untested */
} river_exit_stats_t;

/* Sizes of the four device buffers the caller must allocate for cfg.
 * Shared KV cache layout (bf16): K then V, each [L][max_batch][Hkv][max_seq][Dh],
 * i.e. L*2*Hkv*Dh*2 bytes per token and row; exit layers add no KV bytes.
 * That is the single shared cache of the lead page's section 3 (an exit layer
 * writes the slot of the layer it copies); section 6's peak-memory figures at
 * 16K and 64K tokens grow by exactly this per-token amount for the original
 * model and for the exit scheme alike (131,072 B per token at the Llama-3.1-8B
 * shape).  Returns RIVER_E_INVALID_ARG / RIVER_E_UNIMPLEMENTED for unusable
 * shapes. */
int river_query_sizes(const river_config *cfg, river_sizes *out);

/* Byte offsets, inside the exit bank, of one exit linear of one layer.
 * linear: 0 wq, 1 wk, 2 wv, 3 wo, 4 w_gate, 5 w_up, 6 w_down.
 * Packed int4 layout of a linear with N rows and K columns:
 *   codes: uint32 [N][K/8]; word w of row n holds the codes of columns
 *          8w..8w+7: byte i holds column 8w+i in its low nibble and column
 *          8w+i+4 in its high nibble;
 *   sz:    uint32 [N][K/G]; bf16 scale in bits 0..15, bf16 zero in 16..31;
 *   w_hat = (code - zero) * scale.
 * In RIVER_EXIT_COPY mode the bank holds bf16 [N][K] copies instead, each
 * starting at codes_off of the copy layout (pass copy_layout = 1); sz_off is
 * then unused and set to 0. */
int river_exit_bank_offsets(const river_config *cfg, int32_t layer, int32_t linear,
                            int32_t copy_layout, size_t *codes_off, size_t *sz_off);

/* Create a context for the decoder of the lead page's section 3 (backbone
 * layers, one exit layer beside each, one shared KV cache).  exit_bank,
 * kv_cache, workspace, control: device buffers
 * of at least the sizes in `given`, which must be no smaller than what
 * river_query_sizes(cfg) reports (else RIVER_E_BAD_SIZE).  w: backbone weights,
 * borrowed.  hip_stream: a hipStream_t (NULL = the null stream).  Touches no
 * device memory and launches nothing; *out receives the new context. */
int river_init(const river_config *cfg, const river_weights *w, void *exit_bank,
               void *kv_cache, void *workspace, void *control, const river_sizes *given,
               void *hip_stream, river_ctx **out);

/* Build the exit layers (section 3 of the lead page: copy every layer's
 * parameters, then quantise its seven linear matrices to int4; the norm gains
 * stay as they are and are read from the backbone).  Per (row, group of G
 * columns), in float32 with every operation separately rounded:
 *   s = bf16((max - min) / 15), s = 1 if that is 0;  z = bf16(-min / s);
 *   code = clamp(round_half_even(w / s + z), 0, 15).
 * mode RIVER_EXIT_HQQ then refines each group's zero point in the manner of
 * HQQ, the quantiser the lead page names as its default (section 6; the page
 * gives none of its steps): with zf = z, 20 rounds of
 *   q = clamp(round_half_even(w / s + zf), 0, 15);  e = w - (q - zf) s;
 *   we = sign(e) max(|e| - 1/beta, 0);  zf = sum_group(q - (w - we) / s) / G;
 *   beta = beta * 1.01   (beta = 10 to begin with),
 * every operation float32 and separately rounded, the group sum a fixed
 * pairwise tree (the two halves added element-wise, then their halves, down
 * to one value); s stays, z = bf16(zf), and the codes are taken again with
 * the stored s and z.
 * mode RIVER_EXIT_COPY stores exact bf16 copies instead and needs a bank of
 * exit_bank_copy_bytes (else RIVER_E_BAD_SIZE).  Clears the control block and
 * resets the cache position to 0.  May be called again to rebuild. */
int river_build_exit_layers(river_ctx *ctx, int32_t mode);

/* Prefill B prompts of T tokens each (d_tokens: device int32 [B][T]) into
 * positions 0..T-1 of the shared cache, with ONE sequence-level exit decision
 * per layer: the cosine minimum runs over all B*T rows (section 5).  Writes
 * fp32 logits of each row's last position to d_logits [B][vocab] and the greedy
 * token (lowest index on ties) to d_next [B] (int32); either may be NULL.
 * tau must be finite.  1 <= B <= max_batch, 1 <= T <= max_seq; fixes the batch
 * size for the following decode steps.  Requires river_build_exit_layers. */
int river_prefill(river_ctx *ctx, const int32_t *d_tokens, int32_t B, int32_t T, float tau,
                  float *d_logits, int32_t *d_next);

/* One token-level-exit decode step (section 4): d_tokens device int32 [B]
 * (B from the last prefill) are written at the next position; after each
 * backbone layer l < L-1 the batch-minimum cosine is compared with tau on the
 * device and, once it exceeds tau, layers l+1.. run as exit layers.  Outputs
 * as in river_prefill.  RIVER_E_RANGE when the cache is full.
 * With RIVER_OPT_GRAPH on (and a non-default stream) each step is recorded
 * once as a HIP graph per (d_tokens, d_logits, d_next, batch, forced E) and
 * replayed: reuse the same buffers from step to step.  tau is not part of
 * the recording (a step reads it from the control block, written by one
 * small kernel when it differs from the previous pass's), so a tau sweep
 * replays the same graph.  At most 32 recordings are kept; the 33rd
 * distinct buffer triple drops them all. */
int river_decode_step(river_ctx *ctx, const int32_t *d_tokens, float tau, float *d_logits,
                      int32_t *d_next);

/* n_steps decode steps of river_decode_step (section 4) in one call, the
 * tokens fed back on the device (greedy decoding): step i reads its tokens
 * from d_tokens [B] (i = 0) or from row i-1 of d_next, and writes its next
 * tokens to row i of d_next (device int32 [n_steps][B], required).  Every
 * step writes d_logits [B][vocab] (may be NULL), which so holds the last
 * step's logits.  Each step takes its own exit decision; the statistics count
 * every step.  1 <= n_steps <= 64 (else RIVER_E_INVALID_ARG); RIVER_E_RANGE
 * when the cache has fewer than n_steps free positions; RIVER_E_UNIMPLEMENTED
 * for n_steps > 1 under the recompute comparator.  With RIVER_OPT_GRAPH on the
 * n_steps steps are recorded as ONE graph per (buffers, batch, forced E,
 * n_steps): a replay then pays the graph launch once for n_steps steps. */
int river_decode_steps(river_ctx *ctx, int32_t n_steps, const int32_t *d_tokens, float tau,
                       float *d_logits, int32_t *d_next);

/* Copy the statistics to host memory; synchronises the stream.  The
 * histograms of E per prefill and per decode step, and their mean, are the
 * "mean exit layer" statistic the lead page's section 4 reports per tau (E
 * counts backbone layers run, 1..n_layers).  This is the only call that
 * synchronises with the device; the per-layer activations and the cache
 * slots of a pass are read through river_set_record and the caller-owned
 * kv_cache buffer instead of a separate read-back call. */
int river_exit_stats(river_ctx *ctx, river_exit_stats_t *host_out);

/* Options.
 *   RIVER_OPT_GRAPH   0/1: record each decode-step configuration once as a HIP
 *                     graph and replay it (default 1);
 *   RIVER_OPT_FORCE_E -1 (default) to decide with tau, or e in 0..n_layers to
 *                     run layers < e on the backbone and the rest as exit
 *                     layers without testing (e = n_layers: original model,
 *                     e = 0: every layer quantised);
 *   RIVER_OPT_ATTN_CHUNK positions per decode-attention workgroup: 0 (default)
 *                     lets the library choose per shape, else a multiple of
 *                     64 giving at most 512 splits of max_seq;
 *   RIVER_OPT_GEMV    kernel of the linears of decode steps of at most 8
 *                     rows: 1 the dot-product GEMV, 2 the matrix-core GEMV
 *                     wherever the shape allows (group size 64 or 128, K a
 *                     multiple of 256, the step's rows and the load rings
 *                     within 120 KB of LDS), 0 (default) per linear the one
 *                     measured faster (at one or two rows the matrix-core
 *                     GEMV for gate|up, o and down, from three rows on for
 *                     every linear it fits but the LM head at four rows).
 *                     All give the same results up to the fp32 summation
 *                     order;
 *   RIVER_OPT_ATTN    attention kernels: 0 (default) on the matrix cores
 *                     (decode: scores by MFMA; prefill: flash-style causal
 *                     attention with the probabilities split exactly into
 *                     three bf16 terms), 1 all on the vector ALUs (same
 *                     results up to the fp32 summation order). */
enum { RIVER_OPT_GRAPH = 1, RIVER_OPT_FORCE_E = 2, RIVER_OPT_PROFILE = 3, RIVER_OPT_ATTN_CHUNK = 4,
       RIVER_OPT_GEMV = 5, RIVER_OPT_ATTN = 6, RIVER_OPT_KV_STRATEGY = 7 };
/* RIVER_OPT_KV_STRATEGY: what the layers at and past the exit (E .. L-1) do.
 *   RIVER_KV_RIVER (default): they run as their exit layers and write their
 *     K/V into the shared cache (the method, lead page section 3);
 *   speed comparators, four of the earlier fixes for the K/V that an
 *   early-exited token leaves missing (section 2), the logits then coming
 *   from the exit state:
 *   RIVER_KV_MASK: they are skipped; deeper layers of later tokens leave out
 *     the positions whose K/V they do not hold (matrix-core attention only);
 *   RIVER_KV_PROPAGATE: they only compute their K/V from the exit state (their
 *     RMSNorm gain, backbone k and v projections, RoPE), no attention, no MLP;
 *   RIVER_KV_MONO: they are skipped, and a decode step also exits on reaching
 *     the previous pass's E, so the exit layer never increases along the
 *     sequence;
 *   RIVER_KV_RECOMPUTE: they are skipped; when a later decode step runs a
 *     layer, the earlier positions that hold no K/V there run that layer
 *     (backbone) first, as rows of one prefill-style pass, their states kept
 *     in the buffer river_set_kv_state attaches.  One sequence (batch 1); its
 *     steps run eagerly and read the exit layer back to the host (the next
 *     step's launches depend on it).
 * Decode steps of more than 8 rows take only RIVER_KV_RIVER
 * (RIVER_E_UNIMPLEMENTED); the activation record of a skipped layer holds
 * nothing of the pass.  Setting the option starts no sequence: a prefill
 * under the strategy comes before its decode steps. */
enum { RIVER_KV_RIVER = 0, RIVER_KV_MASK = 1, RIVER_KV_PROPAGATE = 2, RIVER_KV_MONO = 3,
       RIVER_KV_RECOMPUTE = 4 };
int river_set_option(river_ctx *ctx, int32_t option, int64_t value);

/* Kernel classes timed when RIVER_OPT_PROFILE is 1 (decode steps then launch
 * eagerly, with a HIP event recorded on the context's stream before and after
 * every kernel). */
enum {
  RIVER_K_BEGIN = 0,   /* control reset + embedding gather               */
  RIVER_K_QKV = 1,     /* decode: RMSNorm + q|k|v GEMV + RoPE + KV write  */
  RIVER_K_ATTN = 2,    /* decode: split-K GQA attention                   */
  RIVER_K_O = 3,       /* decode: o GEMV + residual                       */
  RIVER_K_GATEUP = 4,  /* decode: RMSNorm + gate|up GEMV + SwiGLU         */
  RIVER_K_DOWN = 5,    /* decode: down GEMV + residual + exit test        */
  RIVER_K_LMHEAD = 6,  /* final RMSNorm + LM head GEMV + argmax           */
  RIVER_K_P_NORM = 7,  /* prefill: RMSNorm rows                           */
  RIVER_K_P_GEMM = 8,  /* prefill: MFMA GEMMs                             */
  RIVER_K_P_ATTN = 9,  /* prefill: causal attention                       */
  RIVER_K_P_COS = 10,  /* prefill: sequence-level exit test               */
  RIVER_K_NKINDS = 11
};
typedef struct {
  int64_t launches;    /* kernels of this class timed since the last read  */
  double total_ms;     /* their summed durations (event to event)          */
} river_kernel_time_t;

/* Per-class kernel times accumulated since the previous call (or since
 * profiling was switched on); out has RIVER_K_NKINDS entries.  Synchronises
 * the stream.  RIVER_E_STATE when profiling is off. */
int river_profile_read(river_ctx *ctx, river_kernel_time_t *out);

/* Kernel timing: the mean execution time of one decode kernel class
 * (RIVER_K_QKV .. RIVER_K_DOWN) in the launch configuration of the current
 * batch.  A HIP graph holding that class's launch for every layer, with the
 * parameters a decode step uses, is replayed `reps` times back to back
 * between two events on the context's stream; avg_us = elapsed / (reps *
 * n_layers).  Which layers take the exit copy follows RIVER_OPT_FORCE_E (set
 * it to the mix to be timed; with -1 the exit flag left by the last step
 * decides).  The kernels overwrite the workspace, and the q|k|v kernel the
 * cache slot of the next position, so call it between steps, not inside a
 * sequence whose next step must see the previous step's state unchanged.
 * Needs a context built on a non-default stream and a prefill before it;
 * synchronises the stream. */
int river_time_kernel(river_ctx *ctx, int32_t kind, int32_t reps, double *avg_us);

/* Debug / test entry point: y = x W^T for one linear of one layer, through
 * the same weight-streaming cores the passes use, with a plain fp32 output
 * instead of a fused epilogue: the GEMV for M <= 8 rows; for 9 <= M <= 64 the
 * batched-row MFMA GEMM of decode steps when the context was made for more
 * than 8 rows (max_batch > 8), else the prefill MFMA GEMM, which also takes
 * every M > 64.
 *   linear: as in river_exit_bank_offsets; use_exit: 0 backbone bf16 weights,
 *   1 the exit copy (int4 or bf16 copy, per the built mode);
 *   d_x: device bf16 [M][K]; d_y: device fp32 [M][N].
 * Enqueues one kernel; RIVER_E_STATE before river_build_exit_layers. */
int river_debug_linear(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit,
                       const void *d_x, int32_t M, float *d_y);

/* river_debug_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments, same kernels and the same results, but the
 * batched-row GEMM's split-K partial tiles (9..64 rows on a context made for
 * more than 8 rows) go to a static device array of the library (32 MiB per
 * GPU, held until the process ends) instead of the context's workspace; it
 * calls no allocating routine.  RIVER_E_BAD_SIZE when the partial tiles of
 * the call would exceed that array (not at the Llama-3.1-8B shapes).  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (on different streams or from different threads) race; each call writes
 * every partial tile it reads, so no clearing is needed between calls. */
int river_debug_linear_noalloc(river_ctx *ctx, int32_t layer, int32_t linear, int32_t use_exit,
                               const void *d_x, int32_t M, float *d_y);

/* Activation record, for checking a pass stage by stage (each layer of a
 * reference can then be fed the states this library stored).  When a record
 * buffer is set, every prefill and decode pass copies, after the kernels that
 * produce them, for each layer l in order:
 *   h_in   fp32 [R][d_model]   residual stream entering layer l
 *   q      bf16 [R][Hq*Dh]     queries after RoPE
 *   attn   bf16 [R][Hq*Dh]     attention output
 *   h_mid  fp32 [R][d_model]   residual after the attention block
 *   u      bf16 [R][ffn_dim]   SwiGLU product
 * and finally h_out fp32 [R][d_model], the residual leaving the last layer.
 * R is the number of rows of the pass (B*T for a prefill, B for a decode
 * step); each array starts on a 256-byte boundary.  K/V are in the cache.
 * river_record_bytes gives the size needed for `rows` rows.  Passing a NULL
 * buffer switches recording off.  While it is on, decode steps run eagerly
 * (no graph); a pass with more rows than the buffer holds fails with
 * RIVER_E_BAD_SIZE before launching anything. */
int river_record_bytes(const river_config *cfg, int32_t rows, size_t *bytes);
int river_set_record(river_ctx *ctx, void *d_buf, size_t bytes);

/* State buffer of the recompute comparator (RIVER_KV_RECOMPUTE): device
 * memory of at least max_seq * d_model * 4 bytes, 16-byte aligned, owned by
 * the caller and used until it is replaced or the context is destroyed.  It
 * holds, per position of the one sequence, the fp32 residual stream at the
 * input of the first layer that position holds no K/V for.  NULL detaches it.
 * Attaching or detaching ends the current sequence for the strategy: decode
 * steps under it return RIVER_E_STATE until a prefill under it.  A prefill
 * or decode step under RIVER_KV_RECOMPUTE without a buffer returns
 * RIVER_E_STATE; RIVER_E_BAD_SIZE for a smaller or misaligned buffer. */
int river_set_kv_state(river_ctx *ctx, void *d_buf, size_t bytes);

/* Start a new sequence: position back to 0 (statistics are kept). */
int river_reset(river_ctx *ctx);

/* Release the host context and its graphs (never the borrowed buffers). */
void river_destroy(river_ctx *ctx);

/* Text of a status code (static storage). */
const char *river_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
