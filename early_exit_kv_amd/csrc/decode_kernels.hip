// Decode-step kernels for gfx950: the pass-begin kernel (control reset and
// embedding gather), the weight-streaming GEMV used for every linear layer at
// small batch (backbone bf16 or exit-layer int4, chosen on the device), and the
// split-K GQA decode attention over the shared KV cache.
//
// Method: "River-LLM: Large Language Model Seamless Exit Based on KV Share",
// section 3 (exit layers share the backbone's KV slots), section 4 (batch-min
// state-transition similarity against tau, no re-check after the exit).
#include "device_common.h"

namespace river {

// ===========================================================================
// Pass begin: reset the per-pass control fields, write tau, gather embeddings.
// ===========================================================================
__global__ __launch_bounds__(256) void begin_kernel(BeginParams p) {
  Control *c = p.ctrl;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      c->flag = 0;
      c->force_E = p.force_E;
      c->E = p.force_E >= 0 ? p.force_E : p.n_layers;
      c->tau = p.tau;
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
  hipLaunchKernelGGL(begin_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

__global__ void clear_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
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
// Row mapping of the fused linears.
//   QKV: logical rows come in RoPE pairs: logical 2P, 2P+1 are rows i and
//        i + Dh/2 of head hh, with P = hh*(Dh/2) + i, heads ordered q, k, v.
//   SwiGLU: each workgroup's first half of rows are gate rows, second half the
//        up rows with the same indices.
// ===========================================================================
struct RowRef {
  int seg, row;
  bool valid;
};

template <int EP>
__device__ __forceinline__ RowRef map_row(const GemvParams &p, int blk, int RW, int j) {
  RowRef r;
  if constexpr (EP == kEpQKV) {
    const int L = blk * RW + j;
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
    const int hw = RW >> 1;
    r.seg = j < hw ? 0 : 1;
    r.row = blk * hw + (j < hw ? j : j - hw);
    r.valid = r.row < p.w.seg_rows[0];
  } else {
    r.seg = 0;
    r.row = blk * RW + j;
    r.valid = r.row < p.N;
  }
  return r;
}

// ===========================================================================
// GEMV: y[b][n] = sum_k x[b][k] W[n][k] for B <= M rows.
//   Threads of a workgroup form 256/tpr groups of tpr threads; each group owns
//   R output rows and splits K into 16-byte chunks (8 bf16 weights or 32 int4
//   codes).  The activation slab sits in LDS as bf16 pairs, laid out for the
//   weight format: natural order for bf16, nibble order for int4 (pair j of
//   word w = columns 8w+j and 8w+4+j).
//   int4: a code pair is turned into the bf16 pair (128+q_a, 128+q_b) with one
//   and-or, so sum x(q - z) = dot(x, 128+q) - (128 + z) * sum(x); each 32-code
//   chunk lies in one quantisation group, whose (s, z) finishes the chunk.
// ===========================================================================
constexpr int kXLdsBytes = 48 * 1024;

template <int M, int R, int XS, int EP>
__global__ __launch_bounds__(256) void gemv_kernel(GemvParams p, int tpr, int kslab) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t *xl = reinterpret_cast<uint32_t *>(smem);                      // [M][kslab/2]
  float *xs = reinterpret_cast<float *>(smem + (size_t)M * kslab * 2);     // [M][kslab/32]
  __shared__ float red[4][R * M];
  __shared__ float outv[16][M];   // RW <= 16 rows
  __shared__ float rstd_s[M];
  __shared__ float bred[8];
  __shared__ int last_flag;

  const bool ex = layer_uses_exit(p.ctrl, p.layer);
  const bool q4 = ex && p.exit_mode == RIVER_EXIT_INT4;
  const int groups = 256 / tpr;
  const int RW = groups * R;
  const int g = threadIdx.x / tpr, tl = threadIdx.x % tpr;
  const int blk = blockIdx.x;

  const uint16_t *wrow_bf[R];
  const uint32_t *wrow_q4[R];
  const uint32_t *wrow_sz[R];
  bool rvalid[R];
  const int KW = p.K / 8;        // code words per row
  const int KG = p.K / p.G;      // groups per row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    RowRef rr = map_row<EP>(p, blk, RW, g * R + r);
    rvalid[r] = rr.valid;
    const int row = rr.valid ? rr.row : 0;
    const uint16_t *bf = ex ? p.w.ex_bf[rr.seg] : p.w.bf[rr.seg];
    wrow_bf[r] = bf ? bf + (int64_t)row * p.K : nullptr;
    wrow_q4[r] = q4 ? p.w.q4[rr.seg] + (int64_t)row * KW : nullptr;
    wrow_sz[r] = q4 ? p.w.sz[rr.seg] + (int64_t)row * KG : nullptr;
  }

  // RMSNorm prologue: 1/sqrt(mean(h^2) + eps) per batch row
  if constexpr (XS == kXNorm) {
    for (int b = 0; b < M; ++b) {
      float ss = 0.f;
      if (b < p.B) {
        const float *h = p.h_src + (int64_t)b * p.h_stride;
        for (int k = threadIdx.x * 4; k < p.K; k += 1024) {
          float4 v = *reinterpret_cast<const float4 *>(h + k);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      }
      ss = block_sum(ss, bred);
      if (threadIdx.x == 0) rstd_s[b] = 1.0f / sqrtf(ss / (float)p.K + p.eps);
    }
    __syncthreads();
  }

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < M; ++b) acc[r][b] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += kslab) {
    const int ks = min(kslab, p.K - k0);
    __syncthreads();
    // ---- stage the activation slab as bf16 pairs
    const int npair = ks >> 1;
    for (int idx = threadIdx.x; idx < M * npair; idx += 256) {
      const int b = idx / npair, pr = idx % npair;
      int c0, c1;
      if (q4) { const int w = pr >> 2, j = pr & 3; c0 = 8 * w + j; c1 = c0 + 4; }
      else { c0 = 2 * pr; c1 = c0 + 1; }
      uint32_t v = 0;
      if (b < p.B) {
        if constexpr (XS == kXNorm) {
          const float *h = p.h_src + (int64_t)b * p.h_stride + k0;
          const float rs = rstd_s[b];
          v = pack_bf2(h[c0] * rs * bf2f(p.gain[k0 + c0]), h[c1] * rs * bf2f(p.gain[k0 + c1]));
        } else {
          const uint16_t *x = p.x_src + (int64_t)b * p.x_stride + k0;
          v = (uint32_t)x[c0] | ((uint32_t)x[c1] << 16);
        }
      }
      xl[b * npair + pr] = v;
    }
    if (q4) {
      __syncthreads();
      const int nch = ks >> 5;
      for (int idx = threadIdx.x; idx < M * nch; idx += 256) {
        const int b = idx / nch, ch = idx % nch;
        const uint32_t *src = xl + b * npair + ch * 16;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += bf_lo(src[i]) + bf_hi(src[i]);
        xs[b * (kslab >> 5) + ch] = s;
      }
    }
    __syncthreads();

    if (q4) {
      // ---- int4 exit layer: 32 codes per 16-byte chunk
      const int nch = ks >> 5;
      for (int c = tl; c < nch; c += tpr) {
        uint4 wv[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          wv[r] = rvalid[r] ? *reinterpret_cast<const uint4 *>(wrow_q4[r] + (k0 >> 3) + 4 * c)
                            : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        const int grp = (k0 + 32 * c) / p.G;
        float sc[R], zz[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t szw = rvalid[r] ? wrow_sz[r][grp] : 0u;
          sc[r] = bf_lo(szw);
          zz[r] = 128.0f + bf_hi(szw);
        }
#pragma unroll
        for (int b = 0; b < M; ++b) {
          const uint4 *xp = reinterpret_cast<const uint4 *>(xl + b * npair + c * 16);
          const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
          const float xsum = xs[b * (kslab >> 5) + c];
          const uint32_t xa[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                   x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t wd[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t pairw = ((wd[i] >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
                d = dot2_bf16(pairw, xa[i * 4 + j], d);
              }
            }
            acc[r][b] = fmaf(sc[r], d - zz[r] * xsum, acc[r][b]);
          }
        }
      }
    } else {
      // ---- bf16 weights (backbone, LM head, or exit copies)
      const int nch = ks >> 3;
      for (int c = tl; c < nch; c += tpr) {
        uint4 wv[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          wv[r] = rvalid[r] ? *reinterpret_cast<const uint4 *>(wrow_bf[r] + k0 + 8 * c)
                            : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < M; ++b) {
          const uint4 xv = *reinterpret_cast<const uint4 *>(xl + b * npair + 4 * c);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float d = acc[r][b];
            d = dot2_bf16(wv[r].x, xv.x, d);
            d = dot2_bf16(wv[r].y, xv.y, d);
            d = dot2_bf16(wv[r].z, xv.z, d);
            d = dot2_bf16(wv[r].w, xv.w, d);
            acc[r][b] = d;
          }
        }
      }
    }
  }

  // ---- reduce over the tpr threads of each group
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int b = 0; b < M; ++b) {
      float v = wave_sum(acc[r][b]);
      if (lane == 0) red[wid][r * M + b] = v;
    }
  __syncthreads();
  const int wpg = tpr >> 6;  // waves per group
  for (int idx = threadIdx.x; idx < RW * M; idx += 256) {
    const int j = idx / M, b = idx % M;
    const int gg = j / R, r = j % R;
    float s = 0.f;
    for (int w = 0; w < wpg; ++w) s += red[gg * wpg + w][r * M + b];
    outv[j][b] = s;
  }
  __syncthreads();

  // ---- epilogues
  if constexpr (EP == kEpQKV) {
    const int pos = p.ctrl->pos;
    const int half = p.Dh >> 1;
    for (int idx = threadIdx.x; idx < (RW >> 1) * M; idx += 256) {
      const int pp = idx / M, b = idx % M;
      if (b >= p.B) continue;
      const int L0 = blk * RW + 2 * pp;
      if (L0 >= p.N) continue;
      const int P = L0 >> 1;
      const int hh = P / half, i = P % half;
      float y0 = outv[2 * pp][b], y1 = outv[2 * pp + 1][b];
      if (hh < p.Hq + p.Hkv) {
        const double ang = (double)pos * pow((double)p.rope_theta, -2.0 * i / (double)p.Dh);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = (float)cs, s = (float)sn;
        const float a = y0 * c - y1 * s;
        const float bb = y1 * c + y0 * s;
        y0 = a;
        y1 = bb;
      }
      if (hh < p.Hq) {
        uint16_t *q = p.q_out + (int64_t)b * p.Hq * p.Dh + hh * p.Dh;
        q[i] = f2bf(y0);
        q[i + half] = f2bf(y1);
      } else {
        const bool isk = hh < p.Hq + p.Hkv;
        const int kvh = isk ? hh - p.Hq : hh - p.Hq - p.Hkv;
        uint16_t *base = isk ? p.k_cache : p.v_cache;
        uint16_t *dst = base + (((int64_t)b * p.Hkv + kvh) * p.max_seq + pos) * p.Dh;
        dst[i] = f2bf(y0);
        dst[i + half] = f2bf(y1);
      }
    }
  } else if constexpr (EP == kEpSwiGLU) {
    const int hw = RW >> 1;
    for (int idx = threadIdx.x; idx < hw * M; idx += 256) {
      const int jj = idx / M, b = idx % M;
      const int n = blk * hw + jj;
      if (b >= p.B || n >= p.w.seg_rows[0]) continue;
      const float gt = outv[jj][b], up = outv[hw + jj][b];
      const float si = gt / (1.0f + expf(-gt));
      p.u_out[(int64_t)b * p.u_stride + n] = f2bf(si * up);
    }
  } else if constexpr (EP == kEpResid || EP == kEpResidExit) {
    for (int idx = threadIdx.x; idx < RW * M; idx += 256) {
      const int j = idx % RW, b = idx / RW;
      const int n = blk * RW + j;
      if (b >= p.B || n >= p.N) continue;
      const int64_t o = (int64_t)b * p.h_io_stride + n;
      const float v = p.h_in[o] + outv[j][b];
      p.h_out[o] = v;
      outv[j][b] = v;   // kept for the exit sums below (same thread, same slot)
    }
    if constexpr (EP == kEpResidExit) {
      // every workgroup read the same flag at its start, so all of them agree
      // on whether this layer is tested (no re-check once the exit fired)
      if (p.test_exit && !ex && p.ctrl->force_E < 0) {
        // per-workgroup partial sums of <a,b>, |a|^2, |b|^2 for each batch row,
        // a = layer input, b = layer output, over this workgroup's rows
        __syncthreads();
        for (int b = 0; b < M; ++b) {
          float sd = 0.f, sa = 0.f, sb = 0.f;
          if (b < p.B && threadIdx.x < RW) {
            const int n = blk * RW + threadIdx.x;
            if (n < p.N) {
              const float a = p.h_src[(int64_t)b * p.h_io_stride + n];
              const float v = outv[threadIdx.x][b];
              sd = a * v; sa = a * a; sb = v * v;
            }
          }
          sd = block_sum(sd, bred);
          sa = block_sum(sa, bred);
          sb = block_sum(sb, bred);
          if (threadIdx.x == 0 && b < p.B) {
            float *pp = p.part + (int64_t)blk * kPartFloatsPerWG + 3 * b;
            pp[0] = sd; pp[1] = sa; pp[2] = sb;
          }
        }
        if (arrive_last(&p.ctrl->counters[kCtrExit], gridDim.x, &last_flag)) {
          float mcos = 2.0f;
          for (int b = 0; b < p.B; ++b) {
            float sd = 0.f, sa = 0.f, sb = 0.f;
            for (int w = threadIdx.x; w < (int)gridDim.x; w += 256) {
              const float *pp = p.part + (int64_t)w * kPartFloatsPerWG + 3 * b;
              sd += pp[0]; sa += pp[1]; sb += pp[2];
            }
            sd = block_sum(sd, bred);
            sa = block_sum(sa, bred);
            sb = block_sum(sb, bred);
            const float den = fmaxf(sqrtf(sa) * sqrtf(sb), 1e-8f);
            float cs = sd / den;
            cs = fminf(fmaxf(cs, -1.0f), 1.0f);
            mcos = fminf(mcos, cs);
          }
          if (threadIdx.x == 0) {
            Control *c = p.ctrl;
            if (c->force_E < 0 && c->flag == 0) {
              c->trace[p.layer] = mcos;
              if (mcos > c->tau) {
                c->flag = 1;
                c->E = p.layer + 1;
              }
            }
          }
        }
      }
    }
  } else if constexpr (EP == kEpLogits) {
    for (int idx = threadIdx.x; idx < RW * M; idx += 256) {
      const int j = idx % RW, b = idx / RW;
      const int n = blk * RW + j;
      if (b >= p.B || n >= p.N) continue;
      const float v = outv[j][b];
      if (p.logits) p.logits[(int64_t)b * p.vocab + n] = v;
    }
    if (threadIdx.x < M && threadIdx.x < p.B) {
      const int b = threadIdx.x;
      uint64_t best = 0;
      for (int j = 0; j < RW; ++j) {
        const int n = blk * RW + j;
        if (n >= p.N) break;
        const uint64_t key = ((uint64_t)float_order(outv[j][b]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
        best = key > best ? key : best;
      }
      __hip_atomic_fetch_max(control_keys(p.ctrl) + b, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (arrive_last(&p.ctrl->counters[kCtrLogits], gridDim.x, &last_flag)) {
      Control *c = p.ctrl;
      if (threadIdx.x < p.B && p.next) {
        const uint64_t key = __hip_atomic_load(control_keys(c) + threadIdx.x, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        p.next[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      }
      if (threadIdx.x == 0) {
        const int E = c->E;
        c->last_E = E;
        if (p.is_prefill) {
          c->prefill_hist[E] += 1;
          c->n_prefill += 1;
        } else {
          c->decode_hist[E] += 1;
          c->n_decode += 1;
          c->pos += 1;
        }
      }
    }
  }
}

template <int M, int XS, int EP>
static hipError_t gemv_launch_m(const GemvParams &p, hipStream_t s) {
  constexpr int R = 4;
  const int nch4 = p.K / 32;  // int4 chunks per row decide the thread split
  const int tpr = nch4 >= 256 ? 256 : (nch4 >= 128 ? 128 : 64);
  const int RW = (256 / tpr) * R;
  int kslab = kXLdsBytes / (M * 2);
  kslab = kslab / 256 * 256;
  if (kslab > p.K) kslab = p.K;
  const size_t lds = (size_t)M * kslab * 2 + (size_t)M * (kslab / 32) * 4;
  int rows = p.N;
  if (EP == kEpSwiGLU) rows = 2 * p.w.seg_rows[0];
  const int grid = (rows + RW - 1) / RW;
  hipLaunchKernelGGL((gemv_kernel<M, R, XS, EP>), dim3(grid), dim3(256), lds, s, p, tpr, kslab);
  return hipGetLastError();
}

template <int XS, int EP>
static hipError_t gemv_launch_xe(const GemvParams &p, hipStream_t s) {
  if (p.B <= 1) return gemv_launch_m<1, XS, EP>(p, s);
  if (p.B <= 2) return gemv_launch_m<2, XS, EP>(p, s);
  if (p.B <= 4) return gemv_launch_m<4, XS, EP>(p, s);
  return gemv_launch_m<8, XS, EP>(p, s);
}

hipError_t launch_gemv(XSource xs, Epilogue ep, const GemvParams &p, hipStream_t s) {
  if (p.B < 1 || p.B > 8) return hipErrorInvalidValue;
  switch (ep) {
    case kEpQKV: return gemv_launch_xe<kXNorm, kEpQKV>(p, s);
    case kEpSwiGLU: return gemv_launch_xe<kXNorm, kEpSwiGLU>(p, s);
    case kEpResid: return gemv_launch_xe<kXBf16, kEpResid>(p, s);
    case kEpResidExit: return gemv_launch_xe<kXBf16, kEpResidExit>(p, s);
    case kEpLogits: return gemv_launch_xe<kXNorm, kEpLogits>(p, s);
  }
  (void)xs;
  return hipErrorInvalidValue;
}

// ===========================================================================
// Decode attention (GQA, split over positions).  Workgroup (split, kv head, b)
// scores its chunk of positions for the Hq/Hkv query heads that share the kv
// head (one K/V read serves all of them), keeps the chunk's max and sum, and
// the last workgroup of each (b, kv head) merges the chunks.
// ===========================================================================
template <int DH, int GQ>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams p) {
  constexpr int LPP = DH / 8;          // lanes per position (8 bf16 each)
  constexpr int PPP = 256 / LPP;       // positions per pass
  __shared__ float sc[GQ][kAttnChunk];
  __shared__ float accs[PPP][GQ][DH];
  __shared__ float bred[8];
  __shared__ float mstat[GQ], lstat[GQ];
  __shared__ int last_flag;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int n = p.ctrl->pos + 1;
  const int t0 = split * kAttnChunk;
  const int cnt = min(kAttnChunk, n - t0);
  const int slot = threadIdx.x / LPP, ln = threadIdx.x % LPP;
  const int64_t kvbase = (((int64_t)b * p.Hkv + kvh) * p.S) * DH;
  const uint16_t *K = p.k_cache + kvbase;
  const uint16_t *V = p.v_cache + kvbase;

  if (cnt > 0) {
    float qv[GQ][8];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const uint4 u = *reinterpret_cast<const uint4 *>(p.q + ((int64_t)b * p.Hq + kvh * GQ + h) * DH + ln * 8);
      qv[h][0] = bf_lo(u.x); qv[h][1] = bf_hi(u.x); qv[h][2] = bf_lo(u.y); qv[h][3] = bf_hi(u.y);
      qv[h][4] = bf_lo(u.z); qv[h][5] = bf_hi(u.z); qv[h][6] = bf_lo(u.w); qv[h][7] = bf_hi(u.w);
    }
    for (int tt = slot; tt < cnt; tt += PPP) {
      const uint4 u = *reinterpret_cast<const uint4 *>(K + (int64_t)(t0 + tt) * DH + ln * 8);
      const float kf[8] = {bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y),
                           bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w)};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
        d = group_sum(d, LPP);
        if (ln == 0) sc[h][tt] = d * p.scale;
      }
    }
    __syncthreads();
    for (int h = 0; h < GQ; ++h) {
      float v = threadIdx.x < cnt ? sc[h][threadIdx.x] : -INFINITY;
      const float m = block_min(-v, bred);   // max via min of negatives
      const float mx = -m;
      const float e = threadIdx.x < cnt ? expf(v - mx) : 0.f;
      if (threadIdx.x < cnt) sc[h][threadIdx.x] = e;
      const float l = block_sum(e, bred);
      if (threadIdx.x == 0) { mstat[h] = mx; lstat[h] = l; }
    }
    __syncthreads();
    float acc[GQ][8];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    for (int tt = slot; tt < cnt; tt += PPP) {
      const uint4 u = *reinterpret_cast<const uint4 *>(V + (int64_t)(t0 + tt) * DH + ln * 8);
      const float vf[8] = {bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y),
                           bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w)};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float pr = sc[h][tt];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) accs[slot][h][ln * 8 + e] = acc[h][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < GQ * DH; idx += 256) {
      const int h = idx / DH, e = idx % DH;
      float s = 0.f;
      for (int sl = 0; sl < PPP; ++sl) s += accs[sl][h][e];
      float *pp = p.part + (((int64_t)b * p.Hq + kvh * GQ + h) * p.splits + split) * (DH + 2);
      pp[e] = s;
      if (e == 0) { pp[DH] = mstat[h]; pp[DH + 1] = lstat[h]; }
    }
  }
  if (arrive_last(&p.counters[b * p.Hkv + kvh], gridDim.x, &last_flag)) {
    const int nval = (n + kAttnChunk - 1) / kAttnChunk;
    for (int idx = threadIdx.x; idx < GQ * DH; idx += 256) {
      const int h = idx / DH, e = idx % DH;
      const float *base = p.part + (((int64_t)b * p.Hq + kvh * GQ + h) * p.splits) * (DH + 2);
      float mx = -INFINITY;
      for (int sp = 0; sp < nval; ++sp) mx = fmaxf(mx, base[sp * (DH + 2) + DH]);
      float l = 0.f, o = 0.f;
      for (int sp = 0; sp < nval; ++sp) {
        const float f = expf(base[sp * (DH + 2) + DH] - mx);
        l += f * base[sp * (DH + 2) + DH + 1];
        o += f * base[sp * (DH + 2) + e];
      }
      p.out[((int64_t)b * p.Hq + kvh * GQ + h) * DH + e] = f2bf(o / l);
    }
  }
}

template <int DH>
static hipError_t attn_launch_dh(const AttnParams &p, hipStream_t s) {
  dim3 grid(p.splits, p.Hkv, p.B);
  const int gq = p.Hq / p.Hkv;
  switch (gq) {
    case 1: hipLaunchKernelGGL((attn_decode_kernel<DH, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((attn_decode_kernel<DH, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((attn_decode_kernel<DH, 4>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnParams &p, hipStream_t s) {
  switch (p.Dh) {
    case 64: return attn_launch_dh<64>(p, s);
    case 128: return attn_launch_dh<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace river
