// Decode-step kernels for gfx950: the pass-begin kernel (control reset and
// embedding gather), the weight-streaming GEMV used for every linear layer at
// small batch (backbone bf16 or exit-layer int4, chosen on the device), and the
// split-K GQA decode attention over the shared KV cache.
//
// Method: "River-LLM: Large Language Model Seamless Exit Based on KV Share",
// section 3 (exit layers share the backbone's KV slots), section 4 (batch-min
// state-transition similarity against tau, no re-check after the exit).
#include <algorithm>

#include "device_common.h"

namespace river {

// ===========================================================================
// Pass begin: reset the per-pass control fields (and write tau for a
// prefill), gather embeddings.
// ===========================================================================
__global__ __launch_bounds__(256) void begin_kernel(BeginParams p) {
  Control *c = p.ctrl;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      c->flag = 0;
      c->force_E = p.force_E;
      c->E = p.force_E >= 0 ? p.force_E : p.n_layers;
      if (p.write_tau) c->tau = p.tau;
      c->strategy = p.strategy;
      if (p.set_pos >= 0) c->pos = p.set_pos;
    }
    for (int l = threadIdx.x; l < kMaxLayers; l += blockDim.x) c->trace[l] = __builtin_nanf("");
    uint64_t *keys = control_keys(c);
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) keys[b] = 0;
  }
  // embedding gather: 8 bf16 per thread
  const int per_row = p.d / 8;
  const int64_t total = p.rows * per_row;
  for (int64_t i = tid; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row;
    const int k8 = (int)(i % per_row) * 8;
    int tok = p.tokens[r];
    if (tok < 0 || tok >= p.vocab) {
      c->bad_token = 1;
      tok = 0;
    }
    const uint4 v = *reinterpret_cast<const uint4 *>(p.embed + (int64_t)tok * p.d + k8);
    float4 lo = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
    float4 hi = make_float4(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
    float *dst = p.h + r * p.d + k8;
    *reinterpret_cast<float4 *>(dst) = lo;
    *reinterpret_cast<float4 *>(dst + 4) = hi;
  }
}

hipError_t launch_begin(const BeginParams &p, hipStream_t s) {
  int64_t work = p.rows * (p.d / 8);
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  return launch_1(begin_kernel, dim3((unsigned)blocks), dim3(256), p, s);
}

__global__ void set_tau_kernel(Control *c, float tau) { c->tau = tau; }

hipError_t launch_set_tau(Control *c, float tau, hipStream_t s) {
  hipLaunchKernelGGL(set_tau_kernel, dim3(1), dim3(1), 0, s, c, tau);
  return hipGetLastError();
}

__global__ void set_pos_E_kernel(Control *c, int32_t *pos_E, int n) {
  const int E = c->last_E;
  if (n > 0) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) pos_E[i] = E;
  } else if (blockIdx.x == 0 && threadIdx.x == 0) {
    pos_E[c->pos - 1] = E;   // the position the step wrote (pos was advanced)
  }
}

hipError_t launch_set_pos_E(Control *c, int32_t *pos_E, int n, hipStream_t s) {
  const int blocks = n > 0 ? std::min(64, (n + 255) / 256) : 1;
  hipLaunchKernelGGL(set_pos_E_kernel, dim3(blocks), dim3(256), 0, s, c, pos_E, n);
  return hipGetLastError();
}

__global__ void clear_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds,
                         hipStream_t s) {
  return hipLaunchKernel(fn, grid, block, args, lds, s);
}

hipError_t launch_clear(void *p, size_t bytes, hipStream_t s) {
  size_t n = bytes / 4;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, n);
  return hipGetLastError();
}

// ===========================================================================
// GEMV: y[b][n] = sum_k x[b][k] W[n][k] for B <= M batch rows.
//
// Work split: a workgroup is 4 wavefronts; each wavefront owns R consecutive
// logical rows and splits K across its 64 lanes in 16-byte chunks (8 bf16
// weights or 32 int4 codes), with U chunks per lane issued before any of them
// is used.  Workgroups stride over row blocks, so the activation vector is
// staged into LDS once per workgroup.  Logical rows are mapped per fused
// linear: QKV rows come in RoPE pairs (rows i and i + Dh/2 of one head), and
// each wavefront of the gate|up linear owns R/2 gate rows and the R/2 up rows
// with the same indices, so every epilogue is local to its wavefront.
//
// Activations sit in LDS as bf16 pairs, laid out for the weight format:
// natural order for bf16 weights, nibble order for int4 (pair j of word w =
// columns 8w+j and 8w+4+j).  An int4 code pair becomes the bf16 pair
// (128+q_a, 128+q_b) with one and-or, so
//   sum_k x_k (q_k - z) s = s * (dot(x, 128+q) - (128 + z) * sum_k x_k)
// and each 32-code chunk lies inside one quantisation group.
// ===========================================================================
constexpr int kXLdsBytes = 64 * 1024;


struct RowRef {
  int seg, row;
  bool valid;
};

template <int EP>
__device__ __forceinline__ RowRef map_row(const GemvParams &p, int L, int wave_first, int R) {
  RowRef r;
  if constexpr (EP == kEpQKV) {
    const int half = p.Dh >> 1;
    const int P = L >> 1;
    const int hh = P / half, i = P % half;
    const int fused = hh * p.Dh + i + (L & 1) * half;
    r.valid = L < p.N;
    const int qrows = p.Hq * p.Dh, krows = p.Hkv * p.Dh;
    if (fused < qrows) { r.seg = 0; r.row = fused; }
    else if (fused < qrows + krows) { r.seg = 1; r.row = fused - qrows; }
    else { r.seg = 2; r.row = fused - qrows - krows; }
  } else if constexpr (EP == kEpSwiGLU) {
    const int hw = R >> 1, j = L - wave_first;
    r.seg = j < hw ? 0 : 1;
    r.row = (wave_first >> 1) + (j < hw ? j : j - hw);
    r.valid = r.row < p.w.seg_rows[0];
  } else {
    r.seg = 0;
    r.row = L;
    r.valid = L < p.N;
  }
  return r;
}

// Rows per task and chunks per batch of one GEMV launch.
//   R rows per wavefront task (even for the RoPE pairs of QKV and the
//   gate/up halves of SwiGLU); UQ int4 chunks or UB bf16 chunks per lane make
//   one batch of loads.  With two batches in registers per wavefront and two
//   workgroups per CU, a batch of 8-16 KB per wavefront keeps 16-32 MB of
//   weight reads in flight over the chip.  Larger batches (M) take fewer rows
//   so that the accumulators and both buffers stay in registers.
template <int EP, int M> struct GemvTile {
  static constexpr bool wide = EP == kEpResidExit || EP == kEpLogits;   // long rows / many rows
  // (the LM head streams best in 4 KB tasks: one row, four chunks per lane)
  static constexpr int R = wide ? (M >= 8 || EP == kEpLogits ? 1 : 2)
                                : EP == kEpSwiGLU ? (M >= 4 ? 2 : M == 2 ? 4 : 8) : (M >= 8 ? 2 : 4);
  static constexpr int UQ = wide ? (M >= 4 || EP == kEpLogits ? 4 : 8) : (M >= 4 ? 1 : 2);
  static constexpr int UB = UQ;
};
constexpr int kGemvWgsPerCu = 2;

template <int M, int XS, int EP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 8)))
void gemv_kernel(GemvParams p, int kslab, int ntask) {
  constexpr int R = GemvTile<EP, M>::R, UQ = GemvTile<EP, M>::UQ, UB = GemvTile<EP, M>::UB;
  constexpr int UMAX = UQ > UB ? UQ : UB;
  extern __shared__ uint4 smem4[];
  uint32_t *xl = reinterpret_cast<uint32_t *>(smem4);            // [M][kslab/2] bf16 pairs
  float *xs = reinterpret_cast<float *>(xl + M * (kslab >> 1));  // [M][kslab/32] chunk sums
  constexpr int NS = 4 * M;   // prologue sums: M norms, then 3 exit sums per batch row
  __shared__ float pred[4][NS];
  __shared__ float wred[4][R * M][3];
  __shared__ uint64_t wkey[4][R * M];
  __shared__ int last_flag;

  const int lane = threadIdx.x & 63;
  // the wavefront index is uniform: keep it (and all row addresses) in SGPRs
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = p.K, KW = K >> 3, KG = K >> p.gshift;
  Control *ctl = p.ctrl;
  const int half = kslab >> 1;
  // one LDS stage holds all of K for one or two batch rows (K <= 16384)
  const bool single = M <= 2 || K <= kslab;
  const int wstride = gridDim.x * 4;   // wavefront tasks are strided over all wavefronts

  // ---- exit choice as far as it is known before the pending test (if any).
  // Plain loads of uniform addresses: they go through the scalar cache and do
  // not hold up the vector loads issued below.  (Workgroup 0 of a QKV launch
  // may set the flag while others read it; both values lead to the same
  // choice, because every workgroup also takes the pending decision itself.)
  const int flag0 = ctl->flag;
  const int force0 = ctl->force_E;
  const bool pending = EP == kEpQKV && p.path == kPathDevice && p.test_prev && force0 < 0 && flag0 == 0;
  bool ex = flag0 != 0 || (p.layer >= 0 && force0 >= 0 && p.layer >= force0);
  if (p.layer < 0) ex = false;
  if (p.path != kPathDevice) ex = p.path == kPathExit;
  // with the test pending the weights start streaming on a guess: the
  // backbone, unless it lives in host memory (then the exit copy in HBM)
  if (pending) ex = p.remote_bb != 0;
  // past the exit under a comparator strategy: skipped, or (q|k|v) the k and
  // v rows only, from the backbone weights
  const int strat = ctl->strategy;
  const int action = past_exit_action(ctl, p.layer, p.path);
  if constexpr (EP == kEpResid || EP == kEpSwiGLU || EP == kEpResidExit) {
    if (action != kRun) {
      if constexpr (EP == kEpResid) {   // the residual stream passes through
        for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < (int64_t)p.B * p.N;
             idx += (int64_t)gridDim.x * 256) {
          const int64_t o = (idx / p.N) * p.h_io_stride + idx % p.N;
          p.h_out[o] = p.h_in[o];
        }
      }
      return;
    }
  }
  bool kv_only = false;
  if constexpr (EP == kEpQKV) {
    if (action == kSkip) return;
    if (action == kKvOnly) {
      kv_only = true;
      ex = false;
    }
  }
  bool q4 = ex && p.exit_mode == RIVER_EXIT_INT4;

  // Rows of the current task: row indices plus at most two segment bases (the
  // first half of a gate|up task reads gate rows, the second half up rows; the
  // RoPE pairs of a QKV task belong to one head and so to one segment).
  int rowi[R];
  bool rv[R];
  const uint16_t *bfA = nullptr, *bfB = nullptr;
  const uint32_t *qA = nullptr, *qB = nullptr, *zA = nullptr, *zB = nullptr;
  auto seg_base = [&](int sg, const uint16_t *&bf, const uint32_t *&q, const uint32_t *&z) {
    if (sg == 0) { bf = ex ? p.w.ex_bf[0] : p.w.bf[0]; q = p.w.q4[0]; z = p.w.sz[0]; }
    else if (sg == 1) { bf = ex ? p.w.ex_bf[1] : p.w.bf[1]; q = p.w.q4[1]; z = p.w.sz[1]; }
    else { bf = ex ? p.w.ex_bf[2] : p.w.bf[2]; q = p.w.q4[2]; z = p.w.sz[2]; }
  };
  auto setup_rows = [&](int task) {
    const int first = task * R;
    const int seg0 = map_row<EP>(p, first, first, R).seg;
    seg_base(EP == kEpSwiGLU ? 0 : seg0, bfA, qA, zA);
    seg_base(EP == kEpSwiGLU ? 1 : seg0, bfB, qB, zB);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const RowRef rr = map_row<EP>(p, first + r, first, R);
      rv[r] = rr.valid;
      rowi[r] = rr.valid ? rr.row : 0;
    }
  };
  auto second_half = [&](int r) { return EP == kEpSwiGLU && r >= R / 2; };
  // Two register buffers of weights: while one batch is reduced, the loads of
  // the next are in flight.  Every load is issued unconditionally (so the wait
  // before a batch is a fixed count): chunks past the end of a row are clamped
  // to its last chunk, rows past the end of the matrix read row 0, and past
  // the last batch a spare batch is fetched; none of these results is used.
  v4u wv[2][UMAX][R];
  uint32_t zv[2][UQ][R];
  auto load_batch = [&](auto bc, int k0, int nch, int c0) {
    constexpr int bi = decltype(bc)::value;
    if (q4) {
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int c = min(c0 + 64 * u, nch - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t *q = (second_half(r) ? qB : qA) + (int64_t)rowi[r] * KW + (k0 >> 3) + 4 * c;
          const uint32_t *z = (second_half(r) ? zB : zA) + (int64_t)rowi[r] * KG + ((k0 + 32 * c) >> p.gshift);
          wv[bi][u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(q));
          zv[bi][u][r] = *z;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int c = min(c0 + 64 * u, nch - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint16_t *w = (second_half(r) ? bfB : bfA) + (int64_t)rowi[r] * K + k0 + 8 * c;
          wv[bi][u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(w));
        }
      }
    }
  };
  auto nchunks = [&](int ks) { return q4 ? (ks >> 5) : (ks >> 3); };
  auto per_iter = [&]() { return 64 * (q4 ? UQ : UB); };
  float acc[R][M];
  auto compute_batch = [&](auto bc, int nch, int c0) {
    constexpr int bi = decltype(bc)::value;
    if (q4) {
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int c = c0 + 64 * u;
        if (c < nch) {
#pragma unroll
          for (int b = 0; b < M; ++b) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(xl + b * half + c * 16);
            const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
            const float xsum = xs[b * (kslab >> 5) + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              uint32_t pr[4];
              float d = 0.f;
              unpack_word(wv[bi][u][r][0], pr);
              d = dot2_bf16(pr[0], x0.x, d); d = dot2_bf16(pr[1], x0.y, d);
              d = dot2_bf16(pr[2], x0.z, d); d = dot2_bf16(pr[3], x0.w, d);
              unpack_word(wv[bi][u][r][1], pr);
              d = dot2_bf16(pr[0], x1.x, d); d = dot2_bf16(pr[1], x1.y, d);
              d = dot2_bf16(pr[2], x1.z, d); d = dot2_bf16(pr[3], x1.w, d);
              unpack_word(wv[bi][u][r][2], pr);
              d = dot2_bf16(pr[0], x2.x, d); d = dot2_bf16(pr[1], x2.y, d);
              d = dot2_bf16(pr[2], x2.z, d); d = dot2_bf16(pr[3], x2.w, d);
              unpack_word(wv[bi][u][r][3], pr);
              d = dot2_bf16(pr[0], x3.x, d); d = dot2_bf16(pr[1], x3.y, d);
              d = dot2_bf16(pr[2], x3.z, d); d = dot2_bf16(pr[3], x3.w, d);
              const float sc = bf_lo(zv[bi][u][r]);
              const float zo = 128.0f + bf_hi(zv[bi][u][r]);
              acc[r][b] = fmaf(sc, d - zo * xsum, acc[r][b]);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int c = c0 + 64 * u;
        if (c < nch) {
#pragma unroll
          for (int b = 0; b < M; ++b) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xl + b * half + 4 * c);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float d = acc[r][b];
              d = dot2_bf16(wv[bi][u][r][0], xv.x, d);
              d = dot2_bf16(wv[bi][u][r][1], xv.y, d);
              d = dot2_bf16(wv[bi][u][r][2], xv.z, d);
              d = dot2_bf16(wv[bi][u][r][3], xv.w, d);
              acc[r][b] = d;
            }
          }
        }
      }
    }
  };

  // ---- prologue.  Its own loads go first (RMSNorm input rows; for the first
  // kernel of a layer also the previous layer's exit sums), the first weight
  // batch right behind them, and only then does anything wait: the weights
  // stream in while the prologue reduces and stages the activations.
  const int n8 = K >> 3;
  float sums[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) sums[i] = 0.f;
  // the normalised rows are held in registers when M*K/8 <= 256*kHeld
  constexpr int kHeld = 2;
  const bool held = XS == kXNorm && M * n8 <= 256 * kHeld;
  float4 hv[kHeld][2];
  uint4 gv[kHeld];
  if (XS == kXNorm && held) {
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
      const int idx = min((int)threadIdx.x + 256 * j, M * n8 - 1);
      const int b = min(idx / n8, p.B - 1), g8 = idx % n8;
      const float *h = p.h_src + (int64_t)b * p.h_stride + 8 * g8;
      hv[j][0] = *reinterpret_cast<const float4 *>(h);
      hv[j][1] = *reinterpret_cast<const float4 *>(h + 4);
      gv[j] = *reinterpret_cast<const uint4 *>(p.gain + 8 * g8);
    }
  }
  constexpr int kPartHeld = 4;   // exit partials per thread held in registers
  float pv[kPartHeld][3 * M];
  if (pending) {
#pragma unroll
    for (int j = 0; j < kPartHeld; ++j) {
      const int wg = min((int)threadIdx.x + 256 * j, p.part_wgs - 1);
      const float *pp = p.part + (int64_t)wg * kPartFloatsPerWG;
#pragma unroll
      for (int i = 0; i < 3 * M; ++i) pv[j][i] = pp[i];
    }
  }
  // (k|v rows only: the tasks start past the query rows)
  const int kv_task0 = EP == kEpQKV ? (p.Hq * p.Dh) / R : 0;
  int task = blockIdx.x * 4 + wid + (kv_only ? kv_task0 : 0);
  setup_rows(task);
  load_batch(Buf<0>{}, 0, nchunks(min(kslab, K)), lane);

  if constexpr (XS == kXNorm) {
    if (held) {
#pragma unroll
      for (int j = 0; j < kHeld; ++j) {
        const int idx = threadIdx.x + 256 * j;
        if (idx < M * n8 && idx / n8 < p.B) {
          const int b = idx / n8;
          const float4 a0 = hv[j][0], a1 = hv[j][1];
          const float ss = a0.x * a0.x + a0.y * a0.y + a0.z * a0.z + a0.w * a0.w + a1.x * a1.x +
                           a1.y * a1.y + a1.z * a1.z + a1.w * a1.w;
#pragma unroll
          for (int bb = 0; bb < M; ++bb) sums[bb] += bb == b ? ss : 0.f;
        }
      }
    } else {
      for (int idx = threadIdx.x; idx < M * n8; idx += 256) {
        const int b = idx / n8, g8 = idx - b * n8;
        if (b < p.B) {
          const float *h = p.h_src + (int64_t)b * p.h_stride + 8 * g8;
          const float4 a0 = *reinterpret_cast<const float4 *>(h);
          const float4 a1 = *reinterpret_cast<const float4 *>(h + 4);
          const float ss = a0.x * a0.x + a0.y * a0.y + a0.z * a0.z + a0.w * a0.w + a1.x * a1.x +
                           a1.y * a1.y + a1.z * a1.z + a1.w * a1.w;
#pragma unroll
          for (int bb = 0; bb < M; ++bb) sums[bb] += bb == b ? ss : 0.f;
        }
      }
    }
  }
  if (pending) {
#pragma unroll
    for (int j = 0; j < kPartHeld; ++j) {
      if ((int)threadIdx.x + 256 * j < p.part_wgs) {
#pragma unroll
        for (int b = 0; b < M; ++b) {
          if (b < p.B) {
            sums[M + 3 * b] += pv[j][3 * b];
            sums[M + 3 * b + 1] += pv[j][3 * b + 1];
            sums[M + 3 * b + 2] += pv[j][3 * b + 2];
          }
        }
      }
    }
    for (int wg = threadIdx.x + 256 * kPartHeld; wg < p.part_wgs; wg += 256) {
      const float *pp = p.part + (int64_t)wg * kPartFloatsPerWG;
#pragma unroll
      for (int b = 0; b < M; ++b) {
        if (b < p.B) {
          sums[M + 3 * b] += pp[3 * b];
          sums[M + 3 * b + 1] += pp[3 * b + 1];
          sums[M + 3 * b + 2] += pp[3 * b + 2];
        }
      }
    }
  }
  if (XS == kXNorm || pending) {
    if (XS == kXNorm) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float v = wave_sum_uniform(sums[i]);
        if (lane == 0) pred[wid][i] = v;
      }
    }
    if (pending) {
#pragma unroll
      for (int i = M; i < NS; ++i) {
        const float v = wave_sum_uniform(sums[i]);
        if (lane == 0) pred[wid][i] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i) sums[i] = (pred[0][i] + pred[1][i]) + (pred[2][i] + pred[3][i]);
  }
  if (pending) {
    // exit decision of the previous layer (lead page, section 4): the minimum
    // over the batch of cos(layer input, layer output) must exceed tau.  Every
    // workgroup reaches the same result from the same sums; workgroup 0
    // records it.
    float mcos = 2.0f;
#pragma unroll
    for (int b = 0; b < M; ++b) {
      if (b < p.B) {
        const float sd = sums[M + 3 * b], sa = sums[M + 3 * b + 1], sb = sums[M + 3 * b + 2];
        float cs = sd / fmaxf(sqrtf(sa) * sqrtf(sb), 1e-8f);
        cs = fminf(fmaxf(cs, -1.0f), 1.0f);
        mcos = fminf(mcos, cs);
      }
    }
    // (the same value in every lane; readfirstlane lets the compiler know it,
    // so the weight choice that follows stays in scalar registers)
    // (mono: a step also exits on reaching the previous pass's E)
    const bool fired = __builtin_amdgcn_readfirstlane(
                           (mcos > ctl->tau || (strat == kStratMono && p.layer >= ctl->last_E)) ? 1 : 0) != 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      ctl->trace[p.layer - 1] = mcos;
      if (fired) {
        ctl->E = p.layer;
        __hip_atomic_store(&ctl->flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (fired && strat != kStratRiver) {
      // this layer is the first past the exit under a comparator strategy
      if (strat != kStratPropagate) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the guessed loads land first
        return;
      }
      kv_only = true;   // k and v rows only, from the backbone weights
      ex = false;
      q4 = false;
      task += kv_task0;
      setup_rows(task);
      load_batch(Buf<0>{}, 0, nchunks(min(kslab, K)), lane);
    } else if (fired != ex) {  // the guess was wrong: fetch the other weights instead
      ex = fired;
      q4 = ex && p.exit_mode == RIVER_EXIT_INT4;
      setup_rows(task);
      load_batch(Buf<0>{}, 0, nchunks(min(kslab, K)), lane);
    }
  }

  // ---- stage x[:, k0:k0+ks] as bf16 pairs in the order of the weight format,
  //      and the sum of every 32-column chunk for the int4 fold
  auto stage = [&](int k0, int ks) {
    const int m8 = ks >> 3;
    for (int idx = threadIdx.x; idx < M * m8; idx += 256) {
      const int b = idx / m8, g8 = idx - b * m8;
      const int col = k0 + 8 * g8;
      uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;   // natural pairs (0,1) (2,3) (4,5) (6,7)
      float csum = 0.f;
      if (b < p.B) {
        if constexpr (XS == kXNorm) {
          float4 h0, h1;
          uint4 g;
          const int j = (idx - (int)threadIdx.x) >> 8;
          if (held && k0 == 0 && j < kHeld) {
#pragma unroll
            for (int jj = 0; jj < kHeld; ++jj)
              if (jj == j) { h0 = hv[jj][0]; h1 = hv[jj][1]; g = gv[jj]; }
          } else {
            const float *h = p.h_src + (int64_t)b * p.h_stride + col;
            h0 = *reinterpret_cast<const float4 *>(h);
            h1 = *reinterpret_cast<const float4 *>(h + 4);
            g = *reinterpret_cast<const uint4 *>(p.gain + col);
          }
          float ssb = 0.f;
#pragma unroll
          for (int bb = 0; bb < M; ++bb) ssb = bb == b ? sums[bb] : ssb;
          const float rs = 1.0f / sqrtf(ssb / (float)K + p.eps);
          a0 = pack_bf2(h0.x * rs * bf_lo(g.x), h0.y * rs * bf_hi(g.x));
          a1 = pack_bf2(h0.z * rs * bf_lo(g.y), h0.w * rs * bf_hi(g.y));
          a2 = pack_bf2(h1.x * rs * bf_lo(g.z), h1.y * rs * bf_hi(g.z));
          a3 = pack_bf2(h1.z * rs * bf_lo(g.w), h1.w * rs * bf_hi(g.w));
        } else {
          const uint4 v = *reinterpret_cast<const uint4 *>(p.x_src + (int64_t)b * p.x_stride + col);
          a0 = v.x; a1 = v.y; a2 = v.z; a3 = v.w;
        }
        csum = (bf_lo(a0) + bf_hi(a0)) + (bf_lo(a1) + bf_hi(a1)) + (bf_lo(a2) + bf_hi(a2)) +
               (bf_lo(a3) + bf_hi(a3));
      }
      const uint4 o = make_uint4(a0, a1, a2, a3);
      if (q4) {
        // the four items of a 32-column chunk sit in four adjacent lanes
        csum += dpp<kDppXor1>(csum);
        csum += dpp<kDppXor2>(csum);
        if ((g8 & 3) == 0) xs[b * (kslab >> 5) + (g8 >> 2)] = csum;
      }
      *reinterpret_cast<uint4 *>(xl + b * half + 4 * g8) = o;
    }
    __syncthreads();
  };

  // lane-local epilogue state kept across tasks
  float ed = 0.f, ea = 0.f, eb = 0.f;
  uint64_t best = 0;
  const bool exit_sums = (EP == kEpResidExit) && p.test_exit && !ex && force0 < 0;

  // Operands the epilogue reads from memory (the residual row entries, the
  // layer input for the exit sums, the RoPE rotation), fetched with the
  // weights of a batch so that no load is waited for behind the next batch.
  // Indices are clamped into range: lanes without an output read a valid
  // element and ignore it.
  struct EpiIn {
    float a, b;
    float2 cs;
  };
  const int pos = ctl->pos;
  const float *hsrc = exit_sums ? p.h_src : p.h_in;
  auto epi_load = [&](int first) {
    EpiIn e;
    e.a = 0.f;
    e.b = 0.f;
    e.cs = make_float2(1.f, 0.f);
    if constexpr (EP == kEpQKV) {
      const int hd = p.Dh >> 1;
      const int i = ((first + 2 * (lane / M)) >> 1) % hd;
      e.cs = p.rope[(int64_t)pos * hd + i];
    } else if constexpr (EP == kEpResid || EP == kEpResidExit) {
      const int n = min(first + lane / M, p.N - 1), b = min(lane % M, p.B - 1);
      const int64_t o = (int64_t)b * p.h_io_stride + n;
      e.a = p.h_in[o];
      if constexpr (EP == kEpResidExit) e.b = hsrc[o];
    }
    return e;
  };

  auto finish_task = [&](int first, const EpiIn &e) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < M; ++b) acc[r][b] = wave_sum_uniform(acc[r][b]);
    auto pick = [&](int r, int b) {
      float v = 0.f;
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int bb = 0; bb < M; ++bb)
          if (rr == r && bb == b) v = acc[rr][bb];
      return v;
    };
    if constexpr (EP == kEpQKV) {
      if (lane < (R / 2) * M) {
        const int pp = lane / M, b = lane % M;
        const int L0 = first + 2 * pp;
        if (b < p.B && L0 < p.N) {
          const int hd = p.Dh >> 1;
          const int P = L0 >> 1;
          const int hh = P / hd, i = P % hd;
          float y0 = pick(2 * pp, b), y1 = pick(2 * pp + 1, b);
          if (hh < p.Hq + p.Hkv) {
            const float2 cs = e.cs;
            const float a = y0 * cs.x - y1 * cs.y;
            y1 = y1 * cs.x + y0 * cs.y;
            y0 = a;
          }
          if (hh < p.Hq) {
            uint16_t *q = p.q_out + (int64_t)b * p.Hq * p.Dh + hh * p.Dh;
            q[i] = f2bf(y0);
            q[i + hd] = f2bf(y1);
          } else {
            const bool isk = hh < p.Hq + p.Hkv;
            const int kvh = isk ? hh - p.Hq : hh - p.Hq - p.Hkv;
            uint16_t *dst = (isk ? p.k_cache : p.v_cache) +
                            (((int64_t)b * p.Hkv + kvh) * p.max_seq + pos) * p.Dh;
            dst[i] = f2bf(y0);
            dst[i + hd] = f2bf(y1);
          }
        }
      }
    } else if constexpr (EP == kEpSwiGLU) {
      if (lane < (R / 2) * M) {
        const int jj = lane / M, b = lane % M;
        const int n = (first >> 1) + jj;
        if (b < p.B && n < p.w.seg_rows[0]) {
          const float gt = pick(jj, b), up = pick(R / 2 + jj, b);
          p.u_out[(int64_t)b * p.u_stride + n] = f2bf(gt / (1.0f + expf(-gt)) * up);
        }
      }
    } else if constexpr (EP == kEpResid || EP == kEpResidExit) {
      if (lane < R * M) {
        const int r = lane / M, b = lane % M;
        const int n = first + r;
        if (b < p.B && n < p.N) {
          const int64_t o = (int64_t)b * p.h_io_stride + n;
          const float v = e.a + pick(r, b);
          p.h_out[o] = v;
          if (exit_sums) {
            const float a = e.b;
            ed += a * v;
            ea += a * a;
            eb += v * v;
          }
        }
      }
    } else if constexpr (EP == kEpPlain) {
      if (lane < R * M) {
        const int r = lane / M, b = lane % M;
        const int n = first + r;
        if (b < p.B && n < p.N) p.y_out[(int64_t)b * p.y_stride + n] = pick(r, b);
      }
    } else if constexpr (EP == kEpLogits) {
      if (lane < R * M) {
        const int r = lane / M, b = lane % M;
        const int n = first + r;
        if (b < p.B && n < p.N) {
          const float v = pick(r, b);
          if (p.logits) p.logits[(int64_t)b * p.vocab + n] = v;
          const uint64_t key = ((uint64_t)float_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
          best = key > best ? key : best;
        }
      }
    }
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < M; ++b) acc[r][b] = 0.f;
  };

  if (single) {
    // All of K is staged once.  A wavefront walks its batches (one or more
    // per task) with the next batch's loads issued before the current batch
    // is reduced, so its weight stream never stops for the arithmetic.
    stage(0, K);
    const int nch = nchunks(K), pi = per_iter();
    int cur = task, c0 = lane;
    EpiIn epi[2];
    epi[0] = epi_load(task * R);
    zero_acc();
    auto step = [&](auto bc) -> bool {
      constexpr int bi = decltype(bc)::value;
      int nt = cur, nc0 = c0 + pi;
      const bool task_end = nc0 - lane >= nch;
      if (task_end) {
        nt = cur + wstride;
        nc0 = lane;
      }
      setup_rows(nt);                       // rows past the last task read row 0
      load_batch(Buf<1 - bi>{}, 0, nch, nc0);
      epi[1 - bi] = epi_load(nt * R);
      compute_batch(bc, nch, c0);
      if (task_end) {
        finish_task(cur * R, epi[bi]);
        zero_acc();
      }
      cur = nt;
      c0 = nc0;
      return cur < ntask;
    };
    if (task < ntask)
      while (step(Buf<0>{}) && step(Buf<1>{})) {
      }
  } else {
    // several K slabs: every slab is staged by the whole workgroup in turn
    bool prefetched = true;
    for (; task < ntask; task += wstride) {
      if (!prefetched) setup_rows(task);
      zero_acc();
      for (int k0 = 0; k0 < K; k0 += kslab) {
        const int ks = min(kslab, K - k0);
        __syncthreads();
        stage(k0, ks);
        const int nch = nchunks(ks);
        for (int c0 = lane; c0 - lane < nch; c0 += per_iter()) {
          if (!prefetched) load_batch(Buf<0>{}, k0, nch, c0);
          prefetched = false;
          compute_batch(Buf<0>{}, nch, c0);
        }
      }
      finish_task(task * R, epi_load(task * R));
    }
  }

  // ---- per-workgroup tails
  if constexpr (EP == kEpResidExit) {
    if (exit_sums) {
      // partial sums of this workgroup's rows, summed in a fixed order; the next
      // layer's first kernel reads them after the kernel boundary
      if (lane < R * M) {
        wred[wid][lane][0] = ed;
        wred[wid][lane][1] = ea;
        wred[wid][lane][2] = eb;
      }
      __syncthreads();
      if (threadIdx.x < 3 * M) {
        const int b = threadIdx.x / 3, k = threadIdx.x % 3;
        float s = 0.f;
        for (int w = 0; w < 4; ++w)
          for (int r = 0; r < R; ++r) s += wred[w][r * M + b][k];
        if (b < p.B) p.part[(int64_t)blockIdx.x * kPartFloatsPerWG + 3 * b + k] = s;
      }
    }
  } else if constexpr (EP == kEpLogits) {
    if (lane < R * M) wkey[wid][lane] = best;
    __syncthreads();
    if (threadIdx.x < M && threadIdx.x < p.B) {
      const int b = threadIdx.x;
      uint64_t m = 0;
      for (int w = 0; w < 4; ++w)
        for (int r = 0; r < R; ++r) m = wkey[w][r * M + b] > m ? wkey[w][r * M + b] : m;
      __hip_atomic_fetch_max(control_keys(ctl) + b, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (arrive_last(&ctl->counters[kCtrLogits], gridDim.x, &last_flag)) {
      if (threadIdx.x < p.B && p.next) {
        const uint64_t key = __hip_atomic_load(control_keys(ctl) + threadIdx.x, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        p.next[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      }
      if (threadIdx.x == 0) {
        const int E = ctl->E;
        ctl->last_E = E;
        if (p.is_prefill) {
          ctl->prefill_hist[E] += 1;
          ctl->n_prefill += 1;
        } else {
          ctl->decode_hist[E] += 1;
          ctl->n_decode += 1;
          ctl->pos += 1;
        }
      }
    }
  }
}

// ===========================================================================
// Decode GEMV on the matrix cores: y[m][n] = sum_k x[m][k] W[n][k] for the
// B <= 8 rows of a decode step (M = B padded to 1, 2, 4 or 8).
//
// A tile is 16 logical output rows; the four wavefronts of a workgroup split
// its K.  A unit of a wavefront is 128 bytes of each of the tile's 16 rows
// (int4: 256 codes; bf16: 64 columns), fetched by two LDS-DMA loads of 8 rows
// x 128 bytes: whole cache lines, which stream almost as fast as contiguous
// reads, where the MFMA operand order itself (16 rows x 64 bytes per load)
// would not.  Each row's eight 16-byte chunks land XOR-swizzled by the row
// index so that the operand reads below hit distinct banks.  The unit's
// scale/zero words and the epilogue operands of its tile come in by DMA too,
// and every wait is an explicit count of the DMAs issued since.
//   The MFMA 16x16x32 takes the staged activations as A (batch row m = lane
// % 16; rows past M repeat row M-1 and are never read back) and the weights
// as B (tile column n = lane % 16, K quarter lane / 16).  It sums over the K
// quarters itself, so no cross-lane reduction is needed: the four partial
// tiles meet once in LDS at the end of a tile, where the epilogue runs.
//   int4: per group, sum_k x (q - z) s = s * (sum_k x (128+q) - (128+z) sum_k x)
//   with 128+q made by unpack_word and the group sums of x taken at staging.
// Workgroups are persistent over tiles; each wavefront keeps kMvD units in
// flight in its own LDS ring.
// ===========================================================================
constexpr int kMvD = 4;                 // units in flight per wavefront
constexpr int kMvWgsPerCu = 2;
constexpr int kMvHold = 4;              // staging items per thread held in registers
constexpr int kMvPartHeld = 2;          // exit partials per thread held in registers
constexpr int kMvSlotW = 2048;          // weight bytes of a unit (16 rows x 128 B)

// epilogue outputs per batch row of a tile: QKV 8 RoPE pairs, SwiGLU 8 products
template <int EP> constexpr int mv_outs() { return (EP == kEpQKV || EP == kEpSwiGLU) ? 8 : 16; }
// epilogue operands per item fetched with every unit (QKV cos/sin, residual
// h_in, exit test h_in and the layer input)
template <int EP> constexpr int mv_nepi() {
  return EP == kEpQKV ? 2 : EP == kEpResid ? 1 : EP == kEpResidExit ? 2 : 0;
}
// bytes of a ring slot: weights, scale/zero words, epilogue operands, and
// with XR the unit's slice of the M activation rows (256 columns each; at
// least the 1 KB one DMA writes)
template <int EP, int M, bool XR> constexpr int mv_slot() {
  return kMvSlotW + 256 + 256 * mv_nepi<EP>() + (XR ? (M >= 2 ? 512 * M : 1024) : 0);
}
static int mv_slot_bytes(Epilogue ep, int M, bool xr) {
  return kMvSlotW + 256 + 256 * (ep == kEpQKV ? 2 : ep == kEpResid ? 1 : ep == kEpResidExit ? 2 : 0) +
         (xr ? (M >= 2 ? 512 * M : 1024) : 0);
}

// f(Buf<I>{}) for I = I0 .. N-1, unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void for_slots(F &f) {
  if constexpr (I < N) {
    f(Buf<I>{});
    for_slots<I + 1, N>(f);
  }
}

// weight row of logical row L (tile column L % 16 of tile L / 16)
template <int EP>
__device__ __forceinline__ RowRef mv_row(const GemvParams &p, int L) {
  if constexpr (EP == kEpQKV) {
    return map_row<kEpQKV>(p, L, 0, 0);
  } else if constexpr (EP == kEpSwiGLU) {
    // a tile holds 8 gate rows (columns 0..7) and the 8 up rows of the same index
    RowRef r;
    const int j = L & 15;
    r.seg = j < 8 ? 0 : 1;
    r.row = 8 * (L >> 4) + (j & 7);
    r.valid = r.row < p.w.seg_rows[0];
    return r;
  } else {
    RowRef r;
    r.seg = 0;
    r.row = L;
    r.valid = L < p.N;
    return r;
  }
}

// LDS-DMA: lane L writes its 16 (4) bytes at lds + 16 L (lds + 4 L); `lds` is
// wave-uniform.  Issued from inline assembly so that the compiler does not
// wait for every outstanding DMA before each LDS read; the loop waits itself.
__device__ __forceinline__ void dma16(uint32_t lds, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// the same for data read once (weights): non-temporal, so that the stream
// does not push out of L2 what the workgroups of the launch share (the rows)
__device__ __forceinline__ void dma16_nt(uint32_t lds, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XR: the activation rows do not fit LDS whole (bf16 input only); each unit
// then brings its 256-column slice of them through the ring as well, and the
// group sums of x come from one more MFMA against a B operand of ones.
template <int M, int XS, int EP, int G, bool XR>
__global__ __launch_bounds__(256) void mgemv_kernel(GemvParams p, int ntile) {
  static_assert(!XR || XS == kXBf16, "ring-fed rows: bf16 input");
  extern __shared__ uint4 mv_smem[];
  constexpr int OUTS = mv_outs<EP>();
  constexpr int NEPI = mv_nepi<EP>();
  constexpr int kMvSlot = mv_slot<EP, M, XR>();
  constexpr int kOffX = kMvSlotW + 256 + 256 * NEPI;   // activation slice in a slot (XR)
  constexpr int ITEMS = OUTS * M;                  // epilogue items per tile (<= 128)
  constexpr int IM = M < 4 ? M : 4;                // result rows per lane: 4 * (lane / 16) + i
  constexpr int GW = G / 32;                       // int4 code words per lane per group
  constexpr int NGU = 256 / G;                     // int4 groups per unit
  typedef typename WordsT<GW>::T WT;
  const int K = p.K, KG = K / G, xrow = K + 8;
  char *ring = reinterpret_cast<char *>(mv_smem);                 // [4 waves][kMvD][kMvSlot]
  uint16_t *xl = reinterpret_cast<uint16_t *>(ring + 4 * kMvD * kMvSlot);   // [M][K + 8] bf16
  float *xsg = reinterpret_cast<float *>(xl + (XR ? 0 : M * xrow));         // [M][K / G] group sums
  float *red = xsg + (XR ? 0 : M * KG);                           // [2][4][M][16] partial tiles
  // one-row RMSNorm input: the fp32 row and the bf16 gains land here by DMA
  // ahead of the weight units (see the prologue)
  constexpr bool kDmaRow = M == 1 && XS == kXNorm && !XR;
  float *hrow = red + 2 * 4 * M * 16;                             // [K] fp32
  uint16_t *grow = reinterpret_cast<uint16_t *>(hrow + (kDmaRow ? K : 0));   // [K] bf16, padded
                                                                            // to whole 1 KB DMAs
  __shared__ float pred[4][4 * M];
  __shared__ float tred[ITEMS][3];
  __shared__ uint64_t tkey[ITEMS];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qq = lane >> 4, cl = lane & 15;
  const int mrow = cl < M ? cl : M - 1;            // A-operand row of this lane
  Control *ctl = p.ctrl;
  char *wring = ring + wid * kMvD * kMvSlot;       // this wavefront's ring
  const uint32_t wring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)wring);

  // ---- exit choice as far as it is known before the pending test (as in the
  // GEMV above: every workgroup of a QKV launch that has to take the test
  // takes it itself and reaches the same result)
  const int flag0 = ctl->flag;
  const int force0 = ctl->force_E;
  const bool pending = EP == kEpQKV && p.path == kPathDevice && p.test_prev && force0 < 0 && flag0 == 0;
  bool ex = flag0 != 0 || (p.layer >= 0 && force0 >= 0 && p.layer >= force0);
  if (p.layer < 0) ex = false;
  if (p.path != kPathDevice) ex = p.path == kPathExit;
  // while the test is pending the backbone units start streaming on a guess;
  // with the backbone in host memory the weights wait for the decision
  const bool defer = pending && p.remote_bb != 0;
  const bool int4_mode = p.exit_mode == RIVER_EXIT_INT4;
  const int pos = ctl->pos;
  // past the exit under a comparator strategy: skipped, or (q|k|v) the k and
  // v tiles only, from the backbone weights
  const int strat = ctl->strategy;
  const int action = past_exit_action(ctl, p.layer, p.path);
  if constexpr (EP == kEpResid || EP == kEpSwiGLU || EP == kEpResidExit) {
    if (action != kRun) {
      if constexpr (EP == kEpResid) {   // the residual stream passes through
        for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < (int64_t)p.B * p.N;
             idx += (int64_t)gridDim.x * 256) {
          const int64_t o = (idx / p.N) * p.h_io_stride + idx % p.N;
          p.h_out[o] = p.h_in[o];
        }
      }
      return;
    }
  }
  int tbase = 0;   // first tile (k|v only: past the query rows)
  const int kv_tile0 = EP == kEpQKV ? (p.Hq * p.Dh) / 16 : 0;
  if constexpr (EP == kEpQKV) {
    if (action == kSkip) return;
    if (action == kKvOnly) {
      tbase = kv_tile0;
      ex = false;
    }
  }

  // ---- per-thread epilogue state kept across tiles (the down projection has
  // no pending test, so its weight choice is final here)
  float ed = 0.f, ea = 0.f, eb = 0.f;
  uint64_t best = 0;
  const bool exit_sums = (EP == kEpResidExit) && p.test_exit && !ex && force0 < 0;
  const float *hsrc = exit_sums ? p.h_src : p.h_in;
  const int n8 = K >> 3, total = M * n8;
  // batch row of staging item idx < total (M - 1 comparisons instead of an
  // integer division by the run-time row length)
  auto rowof = [&](int idx) {
    int m = 0;
#pragma unroll
    for (int b = 1; b < M; ++b) m += idx >= b * n8 ? 1 : 0;
    return m;
  };

  // One pass for one weight form (Q4: int4 codes; else bf16 backbone or bf16
  // exit copy).  Returns true when the pending test chose the exit layer and
  // the weights this pass started to stream are the wrong ones.
  auto run = [&](auto qc, bool restart) -> bool {
    constexpr bool Q4 = decltype(qc)::value == 1;
    // XR: the unit's activation slice, M rows of CR 16-byte chunks, in NX DMAs
    constexpr int CR = (Q4 ? 256 : 64) / 8;
    constexpr int NX = XR ? (M * CR * 16 + 1023) / 1024 : 0;
    constexpr int NDMA = 2 + (Q4 ? 1 : 0) + NEPI + NX;  // DMAs per unit
    constexpr int UKB = Q4 ? 256 : 64;             // K columns per unit
    const int KU = K / UKB, U = (KU + 3) >> 2;     // units per tile row, per wavefront
    const int my_tiles = (ntile - tbase - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    if (my_tiles <= 0) return false;               // (k|v only: fewer tiles than workgroups)

    // ---- fetch side: the tile being fetched (this lane's two weight rows,
    // its scale row, its epilogue operands) and the next unit (lti, ls)
    int ltile = -1;
    const char *wr0 = nullptr, *wr1 = nullptr;     // weight rows 8h + lane / 8, as bytes
    const uint32_t *zr = nullptr;                  // scale row lane / 4
    const float *e0 = p.h_in, *e1 = p.h_in;        // epilogue operands of item 64 wid + lane
    const int wchunk = 16 * ((lane & 7) ^ (((lane >> 3) >> 1) & 7));   // swizzled chunk, h = 0
    const int wchunk1 = 16 * ((lane & 7) ^ ((((lane >> 3) + 8) >> 1) & 7));
    auto weight_row = [&](int t, int r) -> const char * {
      const RowRef rr = mv_row<EP>(p, t * 16 + r);
      const int row = rr.valid ? rr.row : 0;
      const int sg = rr.seg;
      if constexpr (Q4) {
        const uint32_t *q = sg == 0 ? p.w.q4[0] : sg == 1 ? p.w.q4[1] : p.w.q4[2];
        return reinterpret_cast<const char *>(q + (int64_t)row * (K >> 3));
      } else {
        const uint16_t *b0 = ex ? p.w.ex_bf[0] : p.w.bf[0];
        const uint16_t *b1 = ex ? p.w.ex_bf[1] : p.w.bf[1];
        const uint16_t *b2 = ex ? p.w.ex_bf[2] : p.w.bf[2];
        return reinterpret_cast<const char *>((sg == 0 ? b0 : sg == 1 ? b1 : b2) + (int64_t)row * K);
      }
    };
    auto set_tile = [&](int t) {
      wr0 = weight_row(t, lane >> 3);
      wr1 = weight_row(t, 8 + (lane >> 3));
      if constexpr (Q4) {
        const RowRef rr = mv_row<EP>(p, t * 16 + (lane >> 2));
        const int row = rr.valid ? rr.row : 0;
        const int sg = rr.seg;
        zr = (sg == 0 ? p.w.sz[0] : sg == 1 ? p.w.sz[1] : p.w.sz[2]) + (int64_t)row * KG;
      }
      const int item = 64 * wid + lane;
      const int m = min(item / OUTS, p.B - 1), j = item % OUTS;
      if constexpr (EP == kEpQKV) {
        const int hd = p.Dh >> 1;
        const float *cs = reinterpret_cast<const float *>(p.rope + (int64_t)pos * hd + (t * 8 + j) % hd);
        e0 = cs;
        e1 = cs + 1;
      } else if constexpr (EP == kEpResid || EP == kEpResidExit) {
        const int n = min(t * 16 + j, p.N - 1);
        const int64_t o = (int64_t)m * p.h_io_stride + n;
        e0 = p.h_in + o;
        e1 = hsrc + o;
      }
    };
    int lti = 0, ls = 0;
    auto fetch = [&](auto dc) {
      constexpr int d = decltype(dc)::value;
      const bool past = lti >= my_tiles;             // past the last unit: the last unit again
      const int ti = past ? my_tiles - 1 : lti, s = past ? U - 1 : ls;
      const int t = tbase + (int)blockIdx.x + ti * (int)gridDim.x;
      if (t != ltile) {
        set_tile(t);
        ltile = t;
      }
      const int ku = min(wid * U + s, KU - 1);
      const uint32_t slot = wring_lds + d * kMvSlot;
      dma16_nt(slot, wr0 + ku * 128 + wchunk);
      dma16_nt(slot + 1024, wr1 + ku * 128 + wchunk1);
      if constexpr (Q4) dma4(slot + kMvSlotW, zr + ku * NGU + min(lane & 3, NGU - 1));
      if constexpr (NEPI >= 1) dma4(slot + kMvSlotW + 256, e0);
      if constexpr (NEPI >= 2) dma4(slot + kMvSlotW + 512, e1);
      if constexpr (XR) {
        // 16-byte chunk c of row m lands at chunk CR m + (c ^ m) of the slice,
        // so that the rows of one operand read sit in distinct banks (chunks
        // past the M rows, when a DMA is not full, repeat a valid one)
#pragma unroll
        for (int h = 0; h < NX; ++h) {
          const int P = 64 * h + lane, m = P / CR, c = (P % CR) ^ (m & (CR - 1));
          dma16(slot + kOffX + 1024 * h,
                p.x_src + (int64_t)min(m, p.B - 1) * p.x_stride + ku * (CR * 8) + 8 * (c & (CR - 1)));
        }
      }
      if (++ls == U) {
        ls = 0;
        ++lti;
      }
    };

    // ---- reduce one unit from ring slot d into tot
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
    // weight chunk c (16 bytes) of tile row cl inside a slot
    const int rbase = (cl >> 3) * 1024 + 128 * (cl & 7);
    const int rswz = (cl >> 1) & 7;
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    auto compute = [&](auto dc, int k0) {
      constexpr int d = decltype(dc)::value;
      const char *slot = wring + d * kMvSlot;
      const uint16_t *xa = xl + mrow * xrow + k0;
      // A operand: 8 columns of this lane's row at column kk of the unit
      auto a_op = [&](int kk) -> bf16x8_t {
        if constexpr (XR) {
          constexpr int CRc = (Q4 ? 256 : 64) / 8;
          const int c = kk >> 3;
          return *reinterpret_cast<const bf16x8_t *>(slot + kOffX + 16 * (CRc * mrow + (c ^ (mrow & (CRc - 1)))));
        } else {
          return *reinterpret_cast<const bf16x8_t *>(xa + kk);
        }
      };
      if constexpr (Q4) {
        uint32_t zw[NGU];
#pragma unroll
        for (int g = 0; g < NGU; ++g) zw[g] = reinterpret_cast<const uint32_t *>(slot + kMvSlotW)[4 * cl + g];
#pragma unroll
        for (int g = 0; g < NGU; ++g) {
          // this lane's G/4 codes of group g: chunk (G/64) g + qq / (64/G... ) of row cl
          WT w;
          if constexpr (G == 128) {
            w = *reinterpret_cast<const WT *>(slot + rbase + 16 * ((4 * g + qq) ^ rswz));
          } else {
            w = *reinterpret_cast<const WT *>(slot + rbase + 16 * ((2 * g + (qq >> 1)) ^ rswz) + 8 * (qq & 1));
          }
          f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < GW; ++j) {
            const bf16x8_t af = a_op(g * G + qq * (G / 4) + 8 * j);
            uint32_t pr[4];
            unpack_word(w[j], pr);
            ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                af, __builtin_bit_cast(bf16x8_t, make_uint4(pr[0], pr[1], pr[2], pr[3])), ag, 0, 0, 0);
            if constexpr (XR) as = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ones, as, 0, 0, 0);
          }
          const float sc = bf_lo(zw[g]), zo = 128.0f + bf_hi(zw[g]);
          const int gg = k0 / G + g;
#pragma unroll
          for (int i = 0; i < IM; ++i) {
            const int m = min(4 * qq + i, M - 1);
            const float xs = XR ? as[i] : xsg[m * KG + gg];
            tot[i] = fmaf(sc, ag[i] - zo * xs, tot[i]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t af = a_op(32 * j + 8 * qq);
          const bf16x8_t bw = *reinterpret_cast<const bf16x8_t *>(slot + rbase + 16 * ((4 * j + qq) ^ rswz));
          tot = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bw, tot, 0, 0, 0);
        }
      }
    };

    // ---- the tile epilogue: partial tiles into LDS, then one thread per item
    auto end_tile = [&](auto dc, int ti) {
      constexpr int d = decltype(dc)::value;
      const int par = ti & 1;
      const int t = tbase + (int)blockIdx.x + ti * (int)gridDim.x;
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        const int m = 4 * qq + i;
        if (m < M) red[((par * 4 + wid) * M + m) * 16 + cl] = tot[i];
      }
      tot = f32x4_t{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      if (tid < ITEMS) {
        const int m = tid / OUTS, j = tid % OUTS;
        const float *rb = red + (par * 4 * M + m) * 16;
        auto y = [&](int n) {
          return (rb[n] + rb[M * 16 + n]) + (rb[2 * M * 16 + n] + rb[3 * M * 16 + n]);
        };
        // this thread's epilogue operands, fetched by its own wavefront
        const float *eo = reinterpret_cast<const float *>(wring + d * kMvSlot + kMvSlotW + 256) + lane;
        if constexpr (EP == kEpQKV) {
          const int L0 = t * 16 + 2 * j;
          if (m < p.B && L0 < p.N) {
            const int hd = p.Dh >> 1;
            const int P = L0 >> 1;
            const int hh = P / hd, i = P % hd;
            float y0 = y(2 * j), y1 = y(2 * j + 1);
            if (hh < p.Hq + p.Hkv) {
              const float c = eo[0], sn = eo[64];
              const float a = y0 * c - y1 * sn;
              y1 = y1 * c + y0 * sn;
              y0 = a;
            }
            if (hh < p.Hq) {
              uint16_t *q = p.q_out + (int64_t)m * p.Hq * p.Dh + hh * p.Dh;
              q[i] = f2bf(y0);
              q[i + hd] = f2bf(y1);
            } else {
              const bool isk = hh < p.Hq + p.Hkv;
              const int kvh = isk ? hh - p.Hq : hh - p.Hq - p.Hkv;
              uint16_t *dst = (isk ? p.k_cache : p.v_cache) +
                              (((int64_t)m * p.Hkv + kvh) * p.max_seq + pos) * p.Dh;
              dst[i] = f2bf(y0);
              dst[i + hd] = f2bf(y1);
            }
          }
        } else if constexpr (EP == kEpSwiGLU) {
          const int n = t * 8 + j;
          if (m < p.B && n < p.w.seg_rows[0]) {
            const float gt = y(j), up = y(j + 8);
            p.u_out[(int64_t)m * p.u_stride + n] = f2bf(gt / (1.0f + expf(-gt)) * up);
          }
        } else if constexpr (EP == kEpResid || EP == kEpResidExit) {
          const int n = t * 16 + j;
          if (m < p.B && n < p.N) {
            const int64_t o = (int64_t)m * p.h_io_stride + n;
            const float v = eo[0] + y(j);
            p.h_out[o] = v;
            if (exit_sums) {
              const float a = eo[64];
              ed += a * v;
              ea += a * a;
              eb += v * v;
            }
          }
        } else if constexpr (EP == kEpPlain) {
          const int n = t * 16 + j;
          if (m < p.B && n < p.N) p.y_out[(int64_t)m * p.y_stride + n] = y(j);
        } else if constexpr (EP == kEpLogits) {
          const int n = t * 16 + j;
          if (m < p.B && n < p.N) {
            const float v = y(j);
            if (p.logits) p.logits[(int64_t)m * p.vocab + n] = v;
            const uint64_t key = ((uint64_t)float_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
            best = key > best ? key : best;
          }
        }
        (void)eo;
      }
    };

    // ---- one-row RMSNorm input (kDmaRow): the fp32 row and the gains go to
    // LDS by DMA ahead of the weight units, so that the prologue waits for
    // them alone (s_waitcnt counts the units issued after them) and reduces
    // while the units stream.  Otherwise the prologue's own loads come after
    // the weight DMAs (the compiler's wait for them waits for those DMAs too).
    if constexpr (kDmaRow) {
      if (!restart) {
        const uint32_t hl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)hrow);
        const uint32_t gl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)grow);
        for (int c = wid; c < K / 256; c += 4)       // 1 KB of the row per DMA
          dma16(hl + 1024 * c, p.h_src + 256 * c + 4 * lane);
        for (int c = wid; c < (K + 511) / 512; c += 4) {   // 1 KB of the gains per DMA
          // (a last, partial chunk: lanes past K read the first gains again,
          // into the LDS padding past the row's K entries)
          const int e = 512 * c + 8 * lane;
          dma16(gl + 1024 * c, p.gain + (e < K ? e : 0));
        }
      }
    }
    if (!defer || restart) for_slots<0, kMvD>(fetch);

    if (!restart && !XR) {
      if constexpr (kDmaRow) {
        // this wavefront's row DMAs have landed (the units issued after them
        // may still be in flight), then every other wavefront's
        if (defer) wait_vm<0>();
        else wait_vm<kMvD * NDMA>();
        __syncthreads();
      }
      float4 hv[kMvHold][2];
      uint4 gv[kMvHold], bv[kMvHold];
#pragma unroll
      for (int j = 0; j < kMvHold; ++j) {
        const int idx = min(tid + 256 * j, total - 1);
        const int mr = rowof(idx);
        const int m = min(mr, p.B - 1), g8 = idx - mr * n8;
        if constexpr (kDmaRow) {
          const float *h = hrow + 8 * g8;
          hv[j][0] = *reinterpret_cast<const float4 *>(h);
          hv[j][1] = *reinterpret_cast<const float4 *>(h + 4);
          gv[j] = *reinterpret_cast<const uint4 *>(grow + 8 * g8);
        } else if constexpr (XS == kXNorm) {
          const float *h = p.h_src + (int64_t)m * p.h_stride + 8 * g8;
          hv[j][0] = *reinterpret_cast<const float4 *>(h);
          hv[j][1] = *reinterpret_cast<const float4 *>(h + 4);
          gv[j] = *reinterpret_cast<const uint4 *>(p.gain + 8 * g8);
        } else {
          bv[j] = *reinterpret_cast<const uint4 *>(p.x_src + (int64_t)m * p.x_stride + 8 * g8);
        }
      }
      float pv[kMvPartHeld][3 * M];
      if (pending) {
#pragma unroll
        for (int j = 0; j < kMvPartHeld; ++j) {
          const int wg = min(tid + 256 * j, p.part_wgs - 1);
          const float *pp = p.part + (int64_t)wg * kPartFloatsPerWG;
#pragma unroll
          for (int i = 0; i < 3 * M; ++i) pv[j][i] = pp[i];
        }
      }
      // RMSNorm sums of squares of the batch rows, and the exit partials of
      // the previous layer (pending test)
      float sums[4 * M];
#pragma unroll
      for (int i = 0; i < 4 * M; ++i) sums[i] = 0.f;
      if constexpr (XS == kXNorm) {
#pragma unroll
        for (int j = 0; j < kMvHold; ++j) {
          const int idx = tid + 256 * j;
          const int mi = rowof(idx);
          if (idx < total && mi < p.B) {
            const float4 a0 = hv[j][0], a1 = hv[j][1];
            const float ss = a0.x * a0.x + a0.y * a0.y + a0.z * a0.z + a0.w * a0.w + a1.x * a1.x +
                             a1.y * a1.y + a1.z * a1.z + a1.w * a1.w;
#pragma unroll
            for (int b = 0; b < M; ++b) sums[b] += b == mi ? ss : 0.f;
          }
        }
        // items past the held ones, kMvHold at a time with all their loads
        // issued before any is used (addresses clamped into the rows)
        for (int idx0 = 256 * kMvHold; idx0 < total; idx0 += 256 * kMvHold) {
          float4 ha[kMvHold], hb[kMvHold];
#pragma unroll
          for (int j = 0; j < kMvHold; ++j) {
            const int idx = min(idx0 + 256 * j + tid, total - 1);
            const int mr = rowof(idx);
            const int m = min(mr, p.B - 1), g8 = idx - mr * n8;
            const float *h = p.h_src + (int64_t)m * p.h_stride + 8 * g8;
            ha[j] = *reinterpret_cast<const float4 *>(h);
            hb[j] = *reinterpret_cast<const float4 *>(h + 4);
          }
#pragma unroll
          for (int j = 0; j < kMvHold; ++j) {
            const int idx = idx0 + 256 * j + tid;
            const int mi = rowof(min(idx, total - 1));
            if (idx < total && mi < p.B) {
              const float4 a0 = ha[j], a1 = hb[j];
              const float ss = a0.x * a0.x + a0.y * a0.y + a0.z * a0.z + a0.w * a0.w + a1.x * a1.x +
                               a1.y * a1.y + a1.z * a1.z + a1.w * a1.w;
#pragma unroll
              for (int b = 0; b < M; ++b) sums[b] += b == mi ? ss : 0.f;
            }
          }
        }
      }
      if (pending) {
#pragma unroll
        for (int j = 0; j < kMvPartHeld; ++j) {
          if (tid + 256 * j < p.part_wgs) {
#pragma unroll
            for (int i = 0; i < 3 * M; ++i)
              if (i < 3 * p.B) sums[M + i] += pv[j][i];
          }
        }
        for (int wg = tid + 256 * kMvPartHeld; wg < p.part_wgs; wg += 256) {
          const float *pp = p.part + (int64_t)wg * kPartFloatsPerWG;
#pragma unroll
          for (int i = 0; i < 3 * M; ++i)
            if (i < 3 * p.B) sums[M + i] += pp[i];
        }
      }
      if (XS == kXNorm || pending) {
#pragma unroll
        for (int i = 0; i < 4 * M; ++i) {
          const float v = wave_sum_uniform(sums[i]);
          if (lane == 0) pred[wid][i] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4 * M; ++i) sums[i] = (pred[0][i] + pred[1][i]) + (pred[2][i] + pred[3][i]);
      }
      bool fired = false;
      if (pending) {
        // exit decision of the previous layer (lead page, section 4): the
        // minimum over the batch of cos(layer input, layer output) must exceed
        // tau; workgroup 0 records it
        float mcos = 2.0f;
#pragma unroll
        for (int b = 0; b < M; ++b) {
          if (b < p.B) {
            const float sd = sums[M + 3 * b], sa = sums[M + 3 * b + 1], sb = sums[M + 3 * b + 2];
            float cs = sd / fmaxf(sqrtf(sa) * sqrtf(sb), 1e-8f);
            cs = fminf(fmaxf(cs, -1.0f), 1.0f);
            mcos = fminf(mcos, cs);
          }
        }
        // (uniform over the workgroup; readfirstlane tells the compiler, so the
        // weight choice that follows stays in scalar registers)
        // (mono: a step also exits on reaching the previous pass's E)
        fired = __builtin_amdgcn_readfirstlane(
                    (mcos > ctl->tau || (strat == kStratMono && p.layer >= ctl->last_E)) ? 1 : 0) != 0;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
          ctl->trace[p.layer - 1] = mcos;
          if (fired) {
            ctl->E = p.layer;
            __hip_atomic_store(&ctl->flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }

      // stage x as bf16 rows (zeros past B) with the group sums of each row
      auto put = [&](int idx, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
        const int m = rowof(min(idx, total - 1)), g8 = idx - m * n8;
        float gs = (bf_lo(a0) + bf_hi(a0)) + (bf_lo(a1) + bf_hi(a1)) + (bf_lo(a2) + bf_hi(a2)) +
                   (bf_lo(a3) + bf_hi(a3));
        // the G/8 items of a group sit in G/8 adjacent lanes
        gs = G == 128 ? sum16(gs) : sum8(gs);
        if (idx < total) {
          *reinterpret_cast<uint4 *>(xl + m * xrow + 8 * g8) = make_uint4(a0, a1, a2, a3);
          if (g8 % (G / 8) == 0) xsg[m * KG + g8 / (G / 8)] = gs;
        }
      };
      auto norm8 = [&](int m, float4 h0, float4 h1, uint4 g, uint32_t &a0, uint32_t &a1, uint32_t &a2,
                       uint32_t &a3) {
        float ssb = 0.f;
#pragma unroll
        for (int b = 0; b < M; ++b) ssb = b == m ? sums[b] : ssb;
        const float rs = 1.0f / sqrtf(ssb / (float)K + p.eps);
        a0 = pack_bf2(h0.x * rs * bf_lo(g.x), h0.y * rs * bf_hi(g.x));
        a1 = pack_bf2(h0.z * rs * bf_lo(g.y), h0.w * rs * bf_hi(g.y));
        a2 = pack_bf2(h1.x * rs * bf_lo(g.z), h1.y * rs * bf_hi(g.z));
        a3 = pack_bf2(h1.z * rs * bf_lo(g.w), h1.w * rs * bf_hi(g.w));
      };
#pragma unroll
      for (int j = 0; j < kMvHold; ++j) {
        const int idx = tid + 256 * j;
        const int m = rowof(min(idx, total - 1));
        uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
        if (idx < total && m < p.B) {
          if constexpr (XS == kXNorm) norm8(m, hv[j][0], hv[j][1], gv[j], a0, a1, a2, a3);
          else { a0 = bv[j].x; a1 = bv[j].y; a2 = bv[j].z; a3 = bv[j].w; }
        }
        put(idx, a0, a1, a2, a3);
      }
      // the items past the held ones, kMvHold at a time with all their loads
      // issued before any is used (addresses clamped into the rows; the
      // batch bound is uniform, so every lane of a wave takes part in put)
      for (int idx0 = 256 * kMvHold; idx0 < total; idx0 += 256 * kMvHold) {
        float4 ha[kMvHold], hb[kMvHold];
        uint4 gb[kMvHold];
#pragma unroll
        for (int j = 0; j < kMvHold; ++j) {
          const int idx = min(idx0 + 256 * j + tid, total - 1);
          const int mr = rowof(idx);
          const int m = min(mr, p.B - 1), g8 = idx - mr * n8;
          if constexpr (XS == kXNorm) {
            const float *h = p.h_src + (int64_t)m * p.h_stride + 8 * g8;
            ha[j] = *reinterpret_cast<const float4 *>(h);
            hb[j] = *reinterpret_cast<const float4 *>(h + 4);
            gb[j] = *reinterpret_cast<const uint4 *>(p.gain + 8 * g8);
          } else {
            gb[j] = *reinterpret_cast<const uint4 *>(p.x_src + (int64_t)m * p.x_stride + 8 * g8);
          }
        }
#pragma unroll
        for (int j = 0; j < kMvHold; ++j) {
          if (idx0 + 256 * j < total) {
            const int idx = idx0 + 256 * j + tid;
            const int m = rowof(min(idx, total - 1));
            uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
            if (idx < total && m < p.B) {
              if constexpr (XS == kXNorm) {
                norm8(m, ha[j], hb[j], gb[j], a0, a1, a2, a3);
              } else {
                a0 = gb[j].x; a1 = gb[j].y; a2 = gb[j].z; a3 = gb[j].w;
              }
            }
            put(idx, a0, a1, a2, a3);
          }
        }
      }
      __syncthreads();
      if (fired && !ex) {
        // the units in flight are the backbone's: let them land before the
        // exit pass refills the same slots
        wait_vm<0>();
        return true;
      }
      if (defer) for_slots<0, kMvD>(fetch);   // the test kept the (host-resident) backbone
    }

    // ---- main loop: unit n of the sequence sits in ring slot n % kMvD; the
    // unit being reduced is unit cs of tile iteration cti.  Before a unit is
    // read, only the DMAs of the kMvD - 1 units fetched after it may still
    // be in flight.
    int cti = 0, cs = 0;
    auto step = [&](auto dc) {
      if (cti < my_tiles) {
        wait_vm<(kMvD - 1) * NDMA>();
        const int ku = wid * U + cs;
        if (ku < KU) compute(dc, ku * UKB);        // units past K (short rows) add nothing
        if (cs == U - 1) end_tile(dc, cti);
        if (++cs == U) {
          cs = 0;
          ++cti;
        }
      }
      fetch(dc);
    };
    while (cti < my_tiles) for_slots<0, kMvD>(step);
    // the spare fetches past the end land before the workgroup leaves
    wait_vm<0>();
    return false;
  };

  // one pass on the weights chosen (or guessed); when the pending test
  // decides against the guess, a second pass on the other weights
  const bool q4 = ex && int4_mode;
  if (q4) {
    run(Buf<1>{}, false);
  } else if (run(Buf<0>{}, false)) {
    // the pending test fired: the exit weights instead; under a comparator
    // strategy this layer is the first past the exit (k|v only, or nothing)
    bool again = true;
    if (strat == kStratRiver) ex = true;
    else if (strat == kStratPropagate) tbase = kv_tile0;
    else again = false;
    if (again) {
      if (ex && int4_mode) run(Buf<1>{}, true);
      else run(Buf<0>{}, true);
    }
  }

  // ---- per-workgroup tails
  if constexpr (EP == kEpResidExit) {
    if (exit_sums) {
      // exit-test partial sums of this workgroup's rows in a fixed order; the
      // next layer's first kernel reads them after the kernel boundary
      if (tid < ITEMS) {
        tred[tid][0] = ed;
        tred[tid][1] = ea;
        tred[tid][2] = eb;
      }
      __syncthreads();
      if (tid < 3 * M) {
        const int b = tid / 3, k = tid % 3;
        float s = 0.f;
        for (int j = 0; j < OUTS; ++j) s += tred[b * OUTS + j][k];
        if (b < p.B) p.part[(int64_t)blockIdx.x * kPartFloatsPerWG + 3 * b + k] = s;
      }
    }
  } else if constexpr (EP == kEpLogits) {
    if (tid < ITEMS) tkey[tid] = best;
    __syncthreads();
    if (tid < M && tid < p.B) {
      uint64_t m = 0;
      for (int j = 0; j < OUTS; ++j) m = tkey[tid * OUTS + j] > m ? tkey[tid * OUTS + j] : m;
      __hip_atomic_fetch_max(control_keys(ctl) + tid, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (arrive_last(&ctl->counters[kCtrLogits], gridDim.x, &last_flag)) {
      if (threadIdx.x < p.B && p.next) {
        const uint64_t key = __hip_atomic_load(control_keys(ctl) + threadIdx.x, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        p.next[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      }
      if (threadIdx.x == 0) {
        const int E = ctl->E;
        ctl->last_E = E;
        if (p.is_prefill) {
          ctl->prefill_hist[E] += 1;
          ctl->n_prefill += 1;
        } else {
          ctl->decode_hist[E] += 1;
          ctl->n_decode += 1;
          ctl->pos += 1;
        }
      }
    }
  }
}


static int gemv_kslab(int M, int K) {
  int kslab = kXLdsBytes / (M * 2);
  kslab = kslab / 256 * 256;
  return kslab >= K ? K : kslab;
}

static int mpad(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }

static int num_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
  }
  return n;
}

// LDS bytes of one mgemv workgroup
static size_t mgemv_lds(Epilogue ep, int M, int K, int G, bool xr) {
  // one-row RMSNorm inputs staged by DMA: fp32 row + bf16 gains
  const bool dma_row = M == 1 && !xr && (ep == kEpQKV || ep == kEpSwiGLU || ep == kEpLogits);
  return (size_t)4 * kMvD * mv_slot_bytes(ep, M, xr) +
         (xr ? 0 : (size_t)M * (K + 8) * 2 + (size_t)M * (K / G) * 4) +
         (size_t)2 * 4 * M * 16 * 4 + (dma_row ? (size_t)K * 4 + (size_t)(K + 511) / 512 * 1024 : 0);
}

static int mgemv_ntile(Epilogue ep, const GemvParams &p) {
  if (ep == kEpSwiGLU) return (p.w.seg_rows[0] + 7) / 8;
  return (p.N + 15) / 16;
}

constexpr size_t kMvMaxLds = 120 * 1024;

// bf16 input rows come through the ring with the weights (measured faster
// than staging them whole at every row count, and the only way once they do
// not fit LDS); RMSNorm inputs are staged normalised
static bool mgemv_xr(Epilogue ep, const GemvParams &) {
  return ep == kEpResid || ep == kEpResidExit || ep == kEpPlain;
}

bool mgemv_fits(Epilogue ep, const GemvParams &p) {
  const int M = p.B <= 1 ? 1 : p.B <= 2 ? 2 : p.B <= 4 ? 4 : 8;
  if (p.G != 64 && p.G != 128) return false;
  if (p.K % 256 != 0 || p.K % p.G != 0) return false;
  if (ep == kEpQKV && p.Dh % 16 != 0) return false;
  return mgemv_lds(ep, M, p.K, p.G, mgemv_xr(ep, p)) <= kMvMaxLds;
}

struct MvPlan {
  int grid, ntile;
  size_t lds;
  const void *fn;
};

template <int M, int XS, int EP>
static MvPlan mgemv_plan_t(Epilogue ep, const GemvParams &p) {
  MvPlan g;
  g.ntile = mgemv_ntile(ep, p);
  const bool xr = mgemv_xr(ep, p);
  g.lds = mgemv_lds(ep, M, p.K, p.G, xr);
  if constexpr (XS == kXBf16) {
    if (xr) {
      g.fn = p.G == 64 ? reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 64, true>)
                       : reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 128, true>);
    } else {
      g.fn = p.G == 64 ? reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 64, false>)
                       : reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 128, false>);
    }
  } else {
    g.fn = p.G == 64 ? reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 64, false>)
                     : reinterpret_cast<const void *>(mgemv_kernel<M, XS, EP, 128, false>);
  }
  // 160 KB of LDS per CU, a few KB of it static per workgroup
  const int fit = (int)((160 * 1024) / (g.lds + 4 * 1024));
  const int per_cu = std::max(1, std::min(kMvWgsPerCu, fit));
  g.grid = std::min(g.ntile, per_cu * num_cus());
  return g;
}

template <int XS, int EP>
static MvPlan mgemv_plan_m(Epilogue ep, const GemvParams &p) {
  switch (mpad(p.B)) {
    case 1: return mgemv_plan_t<1, XS, EP>(ep, p);
    case 2: return mgemv_plan_t<2, XS, EP>(ep, p);
    case 4: return mgemv_plan_t<4, XS, EP>(ep, p);
    default: return mgemv_plan_t<8, XS, EP>(ep, p);
  }
}

static MvPlan mgemv_plan(Epilogue ep, const GemvParams &p) {
  switch (ep) {
    case kEpQKV: return mgemv_plan_m<kXNorm, kEpQKV>(ep, p);
    case kEpSwiGLU: return mgemv_plan_m<kXNorm, kEpSwiGLU>(ep, p);
    case kEpResid: return mgemv_plan_m<kXBf16, kEpResid>(ep, p);
    case kEpResidExit: return mgemv_plan_m<kXBf16, kEpResidExit>(ep, p);
    case kEpPlain: return mgemv_plan_m<kXBf16, kEpPlain>(ep, p);
    default: return mgemv_plan_m<kXNorm, kEpLogits>(ep, p);
  }
}

// GEMV choice: mode 1 the dot-product kernel everywhere, mode 2 the
// matrix-core one wherever it fits, mode 0 (default) the one measured faster
// per linear on 8B shapes: at one row the matrix cores for gate|up, o and
// down (q|k|v and the LM head keep the dot-product GEMV, whose arithmetic
// still hides behind its stream there), at two rows for q|k|v too, from three
// rows on for every linear that fits (the dot products grow with the rows,
// the MFMA work does not), except the LM head up to four rows
static bool use_mgemv(Epilogue ep, const GemvParams &p) {
  if (p.gemv_mode == 1 || !mgemv_fits(ep, p)) return false;
  if (p.gemv_mode == 2) return true;
  if (p.B == 1) return ep != kEpQKV && ep != kEpLogits;
  return !(ep == kEpLogits && p.B <= 4);
}

struct GemvPlan {
  int grid, ntask, kslab;
  size_t lds;
  const void *fn;
};

// Wavefront tasks (R rows each) are spread over at most one residency wave of
// workgroups; with several K slabs (large batch) every workgroup takes one
// task group of 4 tasks.
template <int M, int XS, int EP>
static GemvPlan gemv_plan(const GemvParams &p) {
  constexpr int R = GemvTile<EP, M>::R;
  GemvPlan g;
  g.kslab = gemv_kslab(M, p.K);
  g.lds = (size_t)M * g.kslab * 2 + (size_t)M * (g.kslab / 32) * 4;
  const int rows = EP == kEpSwiGLU ? 2 * p.w.seg_rows[0] : p.N;
  g.ntask = (rows + R - 1) / R;
  g.fn = (const void *)gemv_kernel<M, XS, EP>;
  const int wgs = (g.ntask + 3) / 4;
  if (p.K > g.kslab) {
    g.grid = wgs;
    return g;
  }
  static int resident = 0;
  if (!resident) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g.fn, 256, g.lds) != hipSuccess ||
        per_cu < 1)
      per_cu = 2;
    resident = min(per_cu, kGemvWgsPerCu) * num_cus();
  }
  const int per = (wgs + resident - 1) / resident;   // task groups per workgroup
  g.grid = (wgs + per - 1) / per;
  return g;
}

template <int XS, int EP>
static GemvPlan gemv_plan_m(const GemvParams &p) {
  switch (mpad(p.B)) {
    case 1: return gemv_plan<1, XS, EP>(p);
    case 2: return gemv_plan<2, XS, EP>(p);
    case 4: return gemv_plan<4, XS, EP>(p);
    default: return gemv_plan<8, XS, EP>(p);
  }
}

static GemvPlan plan_for(Epilogue ep, const GemvParams &p) {
  switch (ep) {
    case kEpQKV: return gemv_plan_m<kXNorm, kEpQKV>(p);
    case kEpSwiGLU: return gemv_plan_m<kXNorm, kEpSwiGLU>(p);
    case kEpResid: return gemv_plan_m<kXBf16, kEpResid>(p);
    case kEpResidExit: return gemv_plan_m<kXBf16, kEpResidExit>(p);
    case kEpPlain: return gemv_plan_m<kXBf16, kEpPlain>(p);
    default: return gemv_plan_m<kXNorm, kEpLogits>(p);
  }
}

int gemv_grid(Epilogue ep, const GemvParams &p) {
  return use_mgemv(ep, p) ? mgemv_plan(ep, p).grid : plan_for(ep, p).grid;
}

hipError_t launch_gemv(XSource xs, Epilogue ep, const GemvParams &p, hipStream_t s) {
  if (p.B < 1 || p.B > 8 || ep > kEpPlain) return hipErrorInvalidValue;
  // the input form is fixed by the epilogue: q|k|v, gate|up and the LM head
  // normalise fp32 rows (h_src, gain) on the way in; the others read bf16
  // rows (x_src).  A call that asks for the other form, or leaves its input
  // unset, is refused before anything is launched.
  const XSource want = (ep == kEpQKV || ep == kEpSwiGLU || ep == kEpLogits) ? kXNorm : kXBf16;
  if (xs != want) return hipErrorInvalidValue;
  if (want == kXNorm ? (!p.h_src || !p.gain) : !p.x_src) return hipErrorInvalidValue;
  if (use_mgemv(ep, p)) {
    const MvPlan g = mgemv_plan(ep, p);
    int ntile = g.ntile;
    GemvParams pc = p;
    void *args[] = {&pc, &ntile};
    return launch_kernel(g.fn, dim3(g.grid), dim3(256), args, g.lds, s);
  }
  const GemvPlan g = plan_for(ep, p);
  int kslab = g.kslab, ntask = g.ntask;
  GemvParams pc = p;
  void *args[] = {&pc, &kslab, &ntask};
  return launch_kernel(g.fn, dim3(g.grid), dim3(256), args, g.lds, s);
}

// ===========================================================================
// RoPE table (float64 angles, rounded once to float32)
// ===========================================================================
__global__ void rope_table_kernel(float2 *rope, int max_seq, int head_dim, double theta) {
  const int hd = head_dim / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)max_seq * hd) return;
  const int t = (int)(i / hd), j = (int)(i % hd);
  const double ang = (double)t * pow(theta, -2.0 * j / (double)head_dim);
  double sn, cs;
  sincos(ang, &sn, &cs);
  rope[i] = make_float2((float)cs, (float)sn);
}

hipError_t launch_rope_table(float2 *rope, int max_seq, int head_dim, float theta, hipStream_t s) {
  const int64_t n = (int64_t)max_seq * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, rope,
                     max_seq, head_dim, (double)theta);
  return hipGetLastError();
}

// ===========================================================================
// Decode attention (GQA, split over positions).  Workgroup (split, kv head, b)
// covers `chunk` positions in sub-chunks of 64: all K and V loads of a
// sub-chunk are issued before any is used, one K/V read serves the Hq/Hkv
// query heads that share the kv head, and each wavefront keeps its own online
// softmax (running max and sum).  The four wavefronts merge at the end; with
// several splits the last workgroup of each (b, kv head) merges the splits.
// ===========================================================================
int attn_chunk(int max_seq, int batch, int n_kv_heads) {
  const int pairs = batch * n_kv_heads;
  // a workgroup per CU already at one split per (b, kv head): one split,
  // which the matrix-core kernel runs with eight wavefronts and no merge
  // (measured on the 8B shapes at B=32 with 1.2K positions: 29.8 us against
  // 31.9 with two splits)
  if (pairs >= 256) return (max_seq + 2 * kAttnSub - 1) / (2 * kAttnSub) * (2 * kAttnSub);
  // splits per (b, kv head): enough for about 512 workgroups (two per CU),
  // and at least one per 1024 positions so that long caches stream through
  // many workgroups at once; at most 16, as merging more costs more than the
  // extra parallelism brings (measured on 8B shapes: B=1 and B=8 at 1K
  // positions, B=8 at 16K)
  const int target = std::min(16, std::max((512 + pairs - 1) / pairs, (max_seq + 1023) / 1024));
  int chunk = (max_seq + target - 1) / target;
  chunk = (chunk + kAttnSub - 1) / kAttnSub * kAttnSub;
  return chunk < kAttnSub ? kAttnSub : chunk;
}

template <int DH, int GQ>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams p) {
  if (past_exit_action(p.ctrl, p.layer, kPathDevice) != kRun) return;   // (comparators)
  constexpr int LPP = DH / 8;        // lanes per position (8 bf16 each)
  constexpr int PPW = 64 / LPP;      // positions per wavefront per pass (slots)
  constexpr int PPP = 4 * PPW;       // positions per workgroup per pass
  constexpr int NP = kAttnSub / PPP; // passes per sub-chunk
  __shared__ float wm[4][GQ];
  __shared__ float wl[4][PPW][GQ];
  __shared__ __align__(16) float wo[4][PPW][GQ][DH];
  __shared__ int last_flag;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int slot = lane / LPP, ln = lane % LPP;
  // the first sub-chunk's K/V loads do not wait for the position: their
  // addresses stay inside the cache whatever it is, and positions past it are
  // masked once it has arrived
  const int t0 = split * p.chunk;
  const int n = p.ctrl->pos + 1;
  // scores are kept in the base-2 domain: s * log2(e), so that every softmax
  // exponential is one hardware 2^x (exp(a - b) = 2^(a log2 e - b log2 e))
  const float scale2 = p.scale * 1.4426950408889634f;
  const int t1 = min(n, t0 + p.chunk);
  const int64_t kvbase = (((int64_t)b * p.Hkv + kvh) * p.S) * DH + ln * 8;
  const uint16_t *K = p.k_cache + kvbase;
  const uint16_t *V = p.v_cache + kvbase;

  float qv[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const uint4 u =
        *reinterpret_cast<const uint4 *>(p.q + ((int64_t)b * p.Hq + kvh * GQ + h) * DH + ln * 8);
    qv[h][0] = bf_lo(u.x); qv[h][1] = bf_hi(u.x); qv[h][2] = bf_lo(u.y); qv[h][3] = bf_hi(u.y);
    qv[h][4] = bf_lo(u.z); qv[h][5] = bf_hi(u.z); qv[h][6] = bf_lo(u.w); qv[h][7] = bf_hi(u.w);
  }
  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int tend = min(t1, min(t0 + p.chunk, p.S));   // positions this workgroup reads
  // K/V of one sub-chunk in registers, two sub-chunks in flight: the loads of
  // the next are issued before the current one is reduced
  uint4 kr[2][NP], vr[2][NP];
  auto load = [&](auto bc, int sb) {
    constexpr int bi = decltype(bc)::value;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = sb + i * PPP + wid * PPW + slot;
      const int tc = min(t, p.S - 1);
      kr[bi][i] = *reinterpret_cast<const uint4 *>(K + (int64_t)tc * DH);
      vr[bi][i] = *reinterpret_cast<const uint4 *>(V + (int64_t)tc * DH);
    }
  };
  auto reduce = [&](auto bc, int sb) {
    constexpr int bi = decltype(bc)::value;
    bool ok[NP];
    uint4 kv[NP], vv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = sb + i * PPP + wid * PPW + slot;
      ok[i] = t < t1;
      kv[i] = ok[i] ? kr[bi][i] : make_uint4(0, 0, 0, 0);
      vv[i] = ok[i] ? vr[bi][i] : make_uint4(0, 0, 0, 0);
    }
    float s[NP][GQ];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const float kf[8] = {bf_lo(kv[i].x), bf_hi(kv[i].x), bf_lo(kv[i].y), bf_hi(kv[i].y),
                           bf_lo(kv[i].z), bf_hi(kv[i].z), bf_lo(kv[i].w), bf_hi(kv[i].w)};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
        d = LPP == 16 ? sum16(d) : sum8(d);   // the lanes of one position
        s[i][h] = ok[i] ? d * scale2 : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      // running max over every position this wavefront has seen
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < NP; ++i) mx = fmaxf(mx, s[i][h]);
      if (LPP == 8) mx = fmaxf(mx, dpp<kDppRor8>(mx));
      const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 16));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 32));
      const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 48));
      mx = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
      const float mnew = fmaxf(m[h], mx);
      if (mnew == -INFINITY) continue;   // nothing visible yet in this wavefront
      const float corr = exp2_fast(m[h] - mnew);
      l[h] *= corr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= corr;
      m[h] = mnew;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float pr = ok[i] ? exp2_fast(s[i][h] - mnew) : 0.f;
        l[h] += pr;
        const float vf[8] = {bf_lo(vv[i].x), bf_hi(vv[i].x), bf_lo(vv[i].y), bf_hi(vv[i].y),
                             bf_lo(vv[i].z), bf_hi(vv[i].z), bf_lo(vv[i].w), bf_hi(vv[i].w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
  };
  // the first sub-chunk was requested before the position was known (t0 is
  // always a valid position); the last one is reduced without a prefetch
  load(Buf<0>{}, t0);
  for (int sb = t0; sb < tend;) {
    if (sb + kAttnSub >= tend) {
      reduce(Buf<0>{}, sb);
      break;
    }
    load(Buf<1>{}, sb + kAttnSub);
    reduce(Buf<0>{}, sb);
    sb += kAttnSub;
    if (sb + kAttnSub >= tend) {
      reduce(Buf<1>{}, sb);
      break;
    }
    load(Buf<0>{}, sb + kAttnSub);
    reduce(Buf<1>{}, sb);
    sb += kAttnSub;
  }
  // per-slot results to LDS; m is uniform over the wavefront
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) wm[wid][h] = m[h];
  }
  if (ln == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) wl[wid][slot][h] = l[h];
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float4 *dst = reinterpret_cast<float4 *>(&wo[wid][slot][h][ln * 8]);
    dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
  }
  __syncthreads();
  const bool direct = p.splits == 1;
  float *part_base = p.part + ((int64_t)b * p.Hq + kvh * GQ) * p.splits * (DH + 2);
  for (int idx = threadIdx.x; idx < GQ * DH; idx += 256) {
    const int h = idx / DH, e = idx % DH;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, wm[wv][h]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float f = exp2_fast(wm[wv][h] - M);
        float lw = 0.f, ow = 0.f;
#pragma unroll
        for (int sl = 0; sl < PPW; ++sl) {
          lw += wl[wv][sl][h];
          ow += wo[wv][sl][h][e];
        }
        L += f * lw;
        o += f * ow;
      }
    }
    if (direct) {
      p.out[((int64_t)b * p.Hq + kvh * GQ + h) * DH + e] = f2bf(o / L);
    } else {
      float *pp = part_base + ((int64_t)h * p.splits + split) * (DH + 2);
      st_coherent(pp + e, o);
      if (e == 0) {
        st_coherent(pp + DH, M);
        st_coherent(pp + DH + 1, L);
      }
    }
  }
  if (direct) return;
  if (arrive_last(&p.counters[b * p.Hkv + kvh], gridDim.x, &last_flag)) {
    // merge the splits that hold positions, 16 splits per round of loads,
    // with the same running-max rescaling as inside a split
    const int nval = (n + p.chunk - 1) / p.chunk;
    for (int idx = threadIdx.x; idx < GQ * DH; idx += 256) {
      const int h = idx / DH, e = idx % DH;
      const float *base = part_base + (int64_t)h * p.splits * (DH + 2);
      float M = -INFINITY, L = 0.f, O = 0.f;
      for (int s0 = 0; s0 < nval; s0 += 16) {
        float ms[16], ls[16], os[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const bool ok = s0 + u < nval;
          const float *pp = base + (int64_t)(s0 + u) * (DH + 2);
          ms[u] = ok ? ld_coherent(pp + DH) : -INFINITY;
          ls[u] = ok ? ld_coherent(pp + DH + 1) : 0.f;
          os[u] = ok ? ld_coherent(pp + e) : 0.f;
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < 16; ++u) mx = fmaxf(mx, ms[u]);
        if (mx == -INFINITY) continue;
        const float corr = exp2_fast(M - mx);
        L *= corr;
        O *= corr;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float f = exp2_fast(ms[u] - mx);
          L = fmaf(f, ls[u], L);
          O = fmaf(f, os[u], O);
        }
        M = mx;
      }
      p.out[((int64_t)b * p.Hq + kvh * GQ + h) * DH + e] = f2bf(O / L);
    }
  }
}

// ===========================================================================
// Decode attention with the scores on the matrix cores.  Same work split as
// attn_decode_kernel (workgroup = split x kv head x row, the last workgroup
// of a (row, kv head) merges the splits), with NW wavefronts per workgroup
// and sub-chunks of 16 NW positions (NW = 4: 64, as the vector-ALU kernel;
// NW = 8 for a single split, which then writes its result directly).
// Inside a sub-chunk each wavefront owns a block of 16 consecutive positions:
// their K and V rows (16 x Dh bf16, contiguous in the cache) land in LDS by
// DMA, the next sub-chunk's while this one is reduced, each row's 16-byte
// chunks XOR-swizzled by the position so that operand reads hit distinct
// banks.  Scores: one MFMA 16x16x32 per 32 head dims, the GQ query heads as A
// (rows past GQ zero) and the K block as B, so every (head, position) score
// is computed once; the online softmax (base-2 domain, scores pre-scaled by
// log2 e) reduces over the block's 16 positions by DPP.  P then goes through
// LDS to the lanes that accumulate P V: Dh/8 lanes per position, 8 head dims
// each.
// ===========================================================================
template <int DH>
__device__ __forceinline__ int attn_swz(int r) {
  return DH == 128 ? (r & 15) : ((r >> 1) & 7);
}

// MASK (the kv-mask comparator): positions whose pass exited at or before this
// layer hold no K/V here and are left out; their pos_E words come in by DMA
// with each block.
template <int DH, int GQ, bool MASK, int NW>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(AttnParams p) {
  if (past_exit_action(p.ctrl, p.layer, kPathDevice) != kRun) return;   // (comparators)
  constexpr int CPR = DH * 2 / 16;             // 16-byte chunks per position
  constexpr int BLK = 16 * DH * 2;             // bytes of a 16-position K (or V) block
  constexpr int NDK = BLK / 1024;              // DMAs per block
  constexpr int NDMA = 2 * NDK + (MASK ? 1 : 0);   // DMAs per sub-chunk per wavefront
  constexpr int LPP = DH / 8;                  // P V lanes per position
  constexpr int PPW = 64 / LPP;                // positions per P V pass
  constexpr int NPASS = 16 / PPW;              // passes per block
  constexpr int NJ = DH / 32;                  // score MFMAs per block
  constexpr int KVB = 2 * BLK;                 // one buffer: K block then V block
  constexpr int SUB = 16 * NW;                 // positions per sub-chunk (16 per wavefront)
  constexpr int NT = 64 * NW;                  // threads
  // per wavefront two buffers; the split's partial results reuse the space
  __shared__ __align__(16) char kvs[NW * 2 * KVB];
  __shared__ __align__(16) float pl[NW][16][GQ];
  __shared__ float wm[NW][GQ], wl[NW][GQ];
  __shared__ int last_flag;
  __shared__ int32_t pe[NW][2][64];                // MASK: pos_E of a wavefront's block
  static_assert(NW * PPW * GQ * DH * 4 <= NW * 2 * KVB, "the partial results fit the K/V buffers");

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qq = lane >> 4, cl = lane & 15;
  const int slot = lane / LPP, ln = lane % LPP;
  const int t0 = split * p.chunk;
  const int64_t kvbase = ((int64_t)b * p.Hkv + kvh) * p.S * DH;
  const uint16_t *Kc = p.k_cache + kvbase;
  const uint16_t *Vc = p.v_cache + kvbase;
  char *kvw = kvs + wid * 2 * KVB;                 // this wavefront's two buffers
  const uint32_t kvw_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)kvw);

  // DMA of the block of positions base .. base+15 (clamped into the cache;
  // positions past the visible ones are masked later) into buffer bi
  auto fetch = [&](int bi, int sb) {
    const int base = sb + 16 * wid;
#pragma unroll
    for (int h = 0; h < NDK; ++h) {
      const int P = 64 * h + lane, r = P / CPR, c = (P % CPR) ^ attn_swz<DH>(r);
      const int64_t off = (int64_t)min(base + r, p.S - 1) * DH + 8 * c;
      const uint32_t dst = kvw_lds + bi * KVB + 1024 * h;
      dma16_nt(dst, Kc + off);
      dma16_nt(dst + BLK, Vc + off);
    }
    if constexpr (MASK) {
      const uint32_t pl = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)&pe[wid][bi][0]);
      dma4(pl, p.pos_E + min(base + lane, p.S - 1));
    }
  };

  // the first block is requested before the position is known (t0 is always
  // a valid position), then q
  fetch(0, t0);
  bf16x8_t qa[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (cl < GQ)
      u = *reinterpret_cast<const uint4 *>(p.q + ((int64_t)b * p.Hq + kvh * GQ + cl) * DH + 32 * j + 8 * qq);
    qa[j] = __builtin_bit_cast(bf16x8_t, u);
  }
  const int n = p.ctrl->pos + 1;
  const int t1 = min(n, t0 + p.chunk);
  const float scale2 = p.scale * 1.4426950408889634f;

  // softmax state of head i (rows 4 qq + i; heads live in the lanes of qq = 0)
  float m[4], l[4], acc[GQ][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  auto reduce = [&](int bi, int sb) {
    const char *kb = kvw + bi * KVB;
    const char *vb = kb + BLK;
    const int base = sb + 16 * wid;
    // scores of the block: D[head][position], position = lane % 16
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
    const int rs = attn_swz<DH>(cl);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(kb + 16 * (cl * CPR + ((4 * j + qq) ^ rs)));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], kf, sc, 0, 0, 0);
    }
    bool vis = base + cl < t1;
    // (MASK: an earlier position keeps its K/V at this layer only if its
    // pass ran the layer; the current position always does)
    if constexpr (MASK) vis = vis && (base + cl >= n - 1 || pe[wid][bi][cl] > p.layer);
    float corr[GQ];
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      const float s2 = vis ? sc[i] * scale2 : -INFINITY;
      const float mnew = fmaxf(m[i], max16(s2));
      float c = 1.f, pr = 0.f;
      if (mnew != -INFINITY) {
        c = exp2_fast(m[i] - mnew);
        pr = vis ? exp2_fast(s2 - mnew) : 0.f;
      }
      l[i] = l[i] * c + sum16(pr);
      m[i] = mnew;
      if (qq == 0) pl[wid][cl][i] = pr;
      // every lane takes head i's correction from lane 0
      corr[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 0));
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= corr[h];
    // P V: this lane's 8 head dims of position pass * PPW + slot.  Rows past
    // the visible positions have p = 0 but may hold any bits (a cache slot
    // never written, NaN included), so they are zeroed rather than weighted.
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * PPW + slot;
      uint4 v = *reinterpret_cast<const uint4 *>(vb + 16 * (r * CPR + (ln ^ attn_swz<DH>(r))));
      bool rv = base + r < t1;
      if constexpr (MASK) rv = rv && (base + r >= n - 1 || pe[wid][bi][r] > p.layer);
      if (!rv) v = make_uint4(0, 0, 0, 0);
      const float vf[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                           bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
      float pr[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) pr[h] = pl[wid][r][h];
#pragma unroll
      for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
    }
  };

  int bi = 0;
  for (int sb = t0; sb < t1; sb += SUB) {
    if (sb + SUB < t1) {
      fetch(bi ^ 1, sb + SUB);
      wait_vm<NDMA>();
    } else {
      wait_vm<0>();
    }
    reduce(bi, sb);
    bi ^= 1;
  }
  wait_vm<0>();   // the speculative block of an empty split has landed too

  // per-wavefront results: m and l from lane 0, P V partials per slot
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      wm[wid][h] = m[h];
      wl[wid][h] = l[h];
    }
  }
  __syncthreads();                               // every wavefront is done with its buffers
  float *wo = reinterpret_cast<float *>(kvs);    // [NW][PPW][GQ][DH]
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float4 *dst = reinterpret_cast<float4 *>(wo + ((wid * PPW + slot) * GQ + h) * DH + ln * 8);
    dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
  }
  __syncthreads();
  const bool direct = p.splits == 1;
  float *part_base = p.part + ((int64_t)b * p.Hq + kvh * GQ) * p.splits * (DH + 2);
  for (int idx = tid; idx < GQ * DH; idx += NT) {
    const int h = idx / DH, e = idx % DH;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, wm[wv][h]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float f = exp2_fast(wm[wv][h] - M);
        float ow = 0.f;
#pragma unroll
        for (int sl = 0; sl < PPW; ++sl) ow += wo[((wv * PPW + sl) * GQ + h) * DH + e];
        L += f * wl[wv][h];
        o += f * ow;
      }
    }
    if (direct) {
      p.out[((int64_t)b * p.Hq + kvh * GQ + h) * DH + e] = f2bf(o / L);
    } else {
      float *pp = part_base + ((int64_t)h * p.splits + split) * (DH + 2);
      st_coherent(pp + e, o);
      if (e == 0) {
        st_coherent(pp + DH, M);
        st_coherent(pp + DH + 1, L);
      }
    }
  }
  if (direct) return;
  if (arrive_last(&p.counters[b * p.Hkv + kvh], gridDim.x, &last_flag)) {
    // merge the splits that hold positions, 16 splits per round of loads
    const int nval = (n + p.chunk - 1) / p.chunk;
    for (int idx = tid; idx < GQ * DH; idx += NT) {
      const int h = idx / DH, e = idx % DH;
      const float *base = part_base + (int64_t)h * p.splits * (DH + 2);
      float M = -INFINITY, L = 0.f, O = 0.f;
      for (int s0 = 0; s0 < nval; s0 += 16) {
        float ms[16], ls[16], os[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const bool ok = s0 + u < nval;
          const float *pp = base + (int64_t)(s0 + u) * (DH + 2);
          ms[u] = ok ? ld_coherent(pp + DH) : -INFINITY;
          ls[u] = ok ? ld_coherent(pp + DH + 1) : 0.f;
          os[u] = ok ? ld_coherent(pp + e) : 0.f;
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < 16; ++u) mx = fmaxf(mx, ms[u]);
        if (mx == -INFINITY) continue;
        const float corr = exp2_fast(M - mx);
        L *= corr;
        O *= corr;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float f = exp2_fast(ms[u] - mx);
          L = fmaf(f, ls[u], L);
          O = fmaf(f, os[u], O);
        }
        M = mx;
      }
      p.out[((int64_t)b * p.Hq + kvh * GQ + h) * DH + e] = f2bf(O / L);
    }
  }
}

template <int DH, int GQ, bool MASK>
static hipError_t attn_mfma_launch(const AttnParams &p, dim3 grid, hipStream_t s) {
  // one split per (row, kv head) and few of them: eight wavefronts, so that
  // a workgroup keeps twice the positions in flight and no split merge runs
  if (p.nw8) return launch_1(attn_mfma_kernel<DH, GQ, MASK, 8>, grid, dim3(512), p, s);
  return launch_1(attn_mfma_kernel<DH, GQ, MASK, 4>, grid, dim3(256), p, s);
}

template <int DH>
static hipError_t attn_launch_dh(const AttnParams &p, hipStream_t s) {
  dim3 grid(p.splits, p.Hkv, p.B);
  const int gq = p.Hq / p.Hkv;
  if (p.mfma && p.pos_E) {
    switch (gq) {
      case 1: return attn_mfma_launch<DH, 1, true>(p, grid, s);
      case 2: return attn_mfma_launch<DH, 2, true>(p, grid, s);
      case 4: return attn_mfma_launch<DH, 4, true>(p, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.pos_E) return hipErrorInvalidValue;   // the vector-ALU kernel has no mask
  if (p.mfma) {
    switch (gq) {
      case 1: return attn_mfma_launch<DH, 1, false>(p, grid, s);
      case 2: return attn_mfma_launch<DH, 2, false>(p, grid, s);
      case 4: return attn_mfma_launch<DH, 4, false>(p, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.nw8) return hipErrorInvalidValue;
  switch (gq) {
    case 1: return launch_1(attn_decode_kernel<DH, 1>, grid, dim3(256), p, s);
    case 2: return launch_1(attn_decode_kernel<DH, 2>, grid, dim3(256), p, s);
    case 4: return launch_1(attn_decode_kernel<DH, 4>, grid, dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s) {
  if (p.chunk % kAttnSub || p.splits < 1 || p.splits > kMaxAttnSplits) return hipErrorInvalidValue;
  if (p.nw8 && (p.splits != 1 || p.chunk % (2 * kAttnSub))) return hipErrorInvalidValue;
  switch (p.Dh) {
    case 64: return attn_launch_dh<64>(p, s);
    case 128: return attn_launch_dh<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace river
