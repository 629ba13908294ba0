// Prefill kernels for gfx950 (and the batched-decode linears): RMSNorm over
// rows, an MFMA bf16 GEMM whose weight operand is either bf16 or the int4 exit
// copy dequantised on the fly, causal GQA attention over the prompt, and the
// sequence-level exit test (one decision for all B*T prompt rows).
//
// Method: "River-LLM: Large Language Model Seamless Exit Based on KV Share",
// section 5: prefill exits at the sequence level so that every prompt token
// leaves at the same layer and the prompt stays one parallel pass.
#include <algorithm>

#include "device_common.h"

namespace river {


// ===========================================================================
// RMSNorm rows: x[r] = bf16(h[r] / sqrt(mean(h[r]^2) + eps) * gain).
// One workgroup per row; every thread loads its (up to 8) groups of 4 values
// before reducing, so a row costs one round trip to memory.
// ===========================================================================
constexpr int kNormHeld = 8;   // float4 per thread held in registers (d <= 8192)

__global__ __launch_bounds__(256) void rows_norm_kernel(RowsNormParams p) {
  // (state propagation still normalises the exit state for its k and v)
  if (p.ctrl && past_exit_action(p.ctrl, p.layer, p.path) == kSkip) return;
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const float *h = p.h + r * (p.h_stride ? p.h_stride : (int64_t)p.d);
  float4 v[kNormHeld];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int k = 4 * (threadIdx.x + 256 * i);
    v[i] = k < p.d ? *reinterpret_cast<const float4 *>(h + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i)
    ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)p.d + p.eps);
  uint16_t *x = p.x + r * p.d;
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int k = 4 * (threadIdx.x + 256 * i);
    if (k < p.d) {
      const uint2 g = *reinterpret_cast<const uint2 *>(p.gain + k);
      uint2 o;
      o.x = pack_bf2(v[i].x * rs * bf_lo(g.x), v[i].y * rs * bf_hi(g.x));
      o.y = pack_bf2(v[i].z * rs * bf_lo(g.y), v[i].w * rs * bf_hi(g.y));
      *reinterpret_cast<uint2 *>(x + k) = o;
    }
  }
}

hipError_t launch_rows_norm(const RowsNormParams &p, hipStream_t s) {
  if (p.d % 4 || p.d > 4 * 256 * kNormHeld) return hipErrorInvalidValue;
  return launch_1(rows_norm_kernel, dim3((unsigned)p.rows), dim3(256), p, s);
}

__global__ __launch_bounds__(256) void rows_copy_run_kernel(float4 *__restrict__ dst, const float4 *__restrict__ src,
                                                            int64_t n4, const Control *ctrl, int layer, int path) {
  if (past_exit_action(ctrl, layer, path) != kRun) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_rows_copy_run(float *dst, const float *src, int64_t n, const Control *ctrl, int layer,
                                int path, hipStream_t s) {
  if (n % 4 || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16)
    return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(1024, (n4 + 255) / 256));
  hipLaunchKernelGGL(rows_copy_run_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<float4 *>(dst),
                     reinterpret_cast<const float4 *>(src), n4, ctrl, layer, path);
  return hipGetLastError();
}

// ===========================================================================
// Sequence-level exit test: c_r = cos(a_r, b_r) for every row, m = min_r c_r;
// the last workgroup compares m with tau and sets the sticky flag.
// ===========================================================================
__global__ __launch_bounds__(256) void rows_cos_kernel(RowsCosParams p) {
  __shared__ float bred[8];
  __shared__ int last_flag;
  // once the exit fired no deeper layer is tested; every workgroup reads the
  // same flag, so either all of them skip or none does
  if (p.ctrl->flag != 0 || p.ctrl->force_E >= 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  float c = 2.0f;
  if (r < p.rows) {
    const float *a = p.a + r * p.d, *b = p.b + r * p.d;
    float sd = 0.f, sa = 0.f, sb = 0.f;
    for (int k = lane * 4; k < p.d; k += 256) {
      const float4 x = *reinterpret_cast<const float4 *>(a + k);
      const float4 y = *reinterpret_cast<const float4 *>(b + k);
      sd += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      sa += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      sb += y.x * y.x + y.y * y.y + y.z * y.z + y.w * y.w;
    }
    sd = wave_sum(sd); sa = wave_sum(sa); sb = wave_sum(sb);
    c = sd / fmaxf(sqrtf(sa) * sqrtf(sb), 1e-8f);
    c = fminf(fmaxf(c, -1.0f), 1.0f);
  }
  const float m = block_min(c, bred);
  if (threadIdx.x == 0) st_coherent(&p.part[blockIdx.x], m);
  if (arrive_last(&p.ctrl->counters[kCtrRowsCos], gridDim.x, &last_flag)) {
    float mm = 2.0f;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += 256) mm = fminf(mm, ld_coherent(&p.part[i]));
    mm = block_min(mm, bred);
    if (threadIdx.x == 0) {
      Control *ct = p.ctrl;
      if (ct->force_E < 0 && ct->flag == 0) {
        ct->trace[p.layer] = mm;
        if (mm > ct->tau) {
          ct->flag = 1;
          ct->E = p.layer + 1;
        }
      }
    }
  }
}

hipError_t launch_rows_cos_exit(const RowsCosParams &p, hipStream_t s) {
  const int64_t blocks = (p.rows + 3) / 4;
  return launch_1(rows_cos_kernel, dim3((unsigned)blocks), dim3(256), p, s);
}

// ===========================================================================
// End of a decode layer of many rows in one launch: the exit test of the
// layer (c_r = cos(a_r, b_r), m = min_r c_r against tau in the last
// workgroup, as rows_cos_kernel) and the RMSNorm of its output rows b for the
// next layer (as rows_norm_kernel, |b_r|^2 serving both).  One workgroup per
// row; `test` false (forced decisions) leaves the test out.
// ===========================================================================
__global__ __launch_bounds__(256) void rows_cos_norm_kernel(RowsCosParams c, RowsNormParams n, int test) {
  __shared__ float red[4], bred[4];
  __shared__ int last_flag;
  const int64_t r = blockIdx.x;
  const float *a = c.a + r * c.d, *b = c.b + r * c.d;
  float4 va[kNormHeld], vb[kNormHeld];
  float sd = 0.f, sa = 0.f, sb = 0.f;
  // the flag is read once by every workgroup before any can change it (only
  // the last one to arrive sets it), so all of them agree on skipping
  const bool do_test = test && c.ctrl->flag == 0 && c.ctrl->force_E < 0;
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int k = 4 * (threadIdx.x + 256 * i);
    vb[i] = k < c.d ? *reinterpret_cast<const float4 *>(b + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    va[i] = do_test && k < c.d ? *reinterpret_cast<const float4 *>(a + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    sb += vb[i].x * vb[i].x + vb[i].y * vb[i].y + vb[i].z * vb[i].z + vb[i].w * vb[i].w;
    sa += va[i].x * va[i].x + va[i].y * va[i].y + va[i].z * va[i].z + va[i].w * va[i].w;
    sd += va[i].x * vb[i].x + va[i].y * vb[i].y + va[i].z * vb[i].z + va[i].w * vb[i].w;
  }
  sb = block_sum(sb, red);
  // RMSNorm of row b
  const float rs = 1.0f / sqrtf(sb / (float)n.d + n.eps);
  uint16_t *x = n.x + r * n.d;
#pragma unroll
  for (int i = 0; i < kNormHeld; ++i) {
    const int k = 4 * (threadIdx.x + 256 * i);
    if (k < n.d) {
      const uint2 g = *reinterpret_cast<const uint2 *>(n.gain + k);
      uint2 o;
      o.x = pack_bf2(vb[i].x * rs * bf_lo(g.x), vb[i].y * rs * bf_hi(g.x));
      o.y = pack_bf2(vb[i].z * rs * bf_lo(g.y), vb[i].w * rs * bf_hi(g.y));
      *reinterpret_cast<uint2 *>(x + k) = o;
    }
  }
  if (!do_test) return;
  sa = block_sum(sa, red);
  sd = block_sum(sd, red);
  float cs = sd / fmaxf(sqrtf(sa) * sqrtf(sb), 1e-8f);
  cs = fminf(fmaxf(cs, -1.0f), 1.0f);
  if (threadIdx.x == 0) st_coherent(&c.part[blockIdx.x], cs);
  if (arrive_last(&c.ctrl->counters[kCtrRowsCos], gridDim.x, &last_flag)) {
    float mm = 2.0f;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += 256) mm = fminf(mm, ld_coherent(&c.part[i]));
    mm = block_min(mm, bred);
    if (threadIdx.x == 0) {
      Control *ct = c.ctrl;
      ct->trace[c.layer] = mm;
      if (mm > ct->tau) {
        ct->flag = 1;
        ct->E = c.layer + 1;
      }
    }
  }
}

hipError_t launch_rows_cos_norm(const RowsCosParams &c, const RowsNormParams &n, bool test, hipStream_t s) {
  if (n.d % 4 || n.d > 4 * 256 * kNormHeld || n.d != c.d || n.rows != c.rows) return hipErrorInvalidValue;
  if (n.h_stride != 0 && n.h_stride != n.d) return hipErrorInvalidValue;
  const int t = test ? 1 : 0;
  void *args[] = {const_cast<RowsCosParams *>(&c), const_cast<RowsNormParams *>(&n), const_cast<int *>(&t)};
  return launch_kernel(reinterpret_cast<const void *>(rows_cos_norm_kernel), dim3((unsigned)c.rows), dim3(256),
                       args, 0, s);
}

// ===========================================================================
// MFMA GEMM: Y[m][n] = sum_k X[m][k] W[n][k] with v_mfma_f32_16x16x32_bf16.
//   Workgroup tile BM x BN, 4 wavefronts in a 2 x 2 arrangement, k-step 32.
//   bf16 weights feed the MFMA directly.  int4 weights enter as the exact bf16
//   values 128 + q; each quantisation group accumulates on its own and is
//   folded as  acc += s * (acc_g - (128 + z) * sum_k x),  so the exit layer
//   computes sum x (q - z) s like the GEMV does.
//   Columns are mapped like the GEMV's rows (RoPE pairs for QKV, gate/up
//   halves for SwiGLU) so that the epilogue sees matching outputs together.
// ===========================================================================
constexpr int kBK = 32;
constexpr int kLdsPad = 8;  // bf16 elements of padding per LDS row

template <int EP>
__device__ __forceinline__ void map_col(const GemmParams &p, int col_blk, int BN, int j, int &seg,
                                        int &row, bool &valid) {
  if constexpr (EP == kEpQKV) {
    const int L = col_blk * BN + j;
    const int half = p.Dh >> 1;
    const int P = L >> 1;
    const int hh = P / half, i = P % half;
    const int fused = hh * p.Dh + i + (L & 1) * half;
    valid = L < p.N;
    const int qrows = p.Hq * p.Dh, krows = p.Hkv * p.Dh;
    if (fused < qrows) { seg = 0; row = fused; }
    else if (fused < qrows + krows) { seg = 1; row = fused - qrows; }
    else { seg = 2; row = fused - qrows - krows; }
  } else if constexpr (EP == kEpSwiGLU) {
    const int hw = BN >> 1;
    seg = j < hw ? 0 : 1;
    row = col_blk * hw + (j < hw ? j : j - hw);
    valid = row < p.w.seg_rows[0];
  } else {
    seg = 0;
    row = col_blk * BN + j;
    valid = row < p.N;
  }
}

// Epilogue of one finished tile: Cs holds rows x BN results (row stride cs)
// for rows m0.. and column block colblk (columns mapped as map_col<EP> says).
template <int EP, int BN, int NTHR = 256>
__device__ void tile_epilogue(const GemmParams &p, const float *Cs, int cs, int BM, int64_t m0,
                              int colblk) {
  const int tid = threadIdx.x;
  if constexpr (EP == kEpQKV) {
    const int half = p.Dh >> 1;
    for (int idx = tid; idx < BM * (BN / 2); idx += NTHR) {
      const int r = idx / (BN / 2), pp = idx % (BN / 2);
      const int64_t m = m0 + r;
      const int L0 = colblk * BN + 2 * pp;
      if (m >= p.M || L0 >= p.N) continue;
      int b, t;
      if (p.T > 0) { b = (int)(m / p.T); t = (int)(m % p.T) + p.start; }
      else { b = (int)m; t = p.ctrl->pos; }
      const int P = L0 >> 1;
      const int hh = P / half, i = P % half;
      float y0 = Cs[r * cs + (2 * pp)], y1 = Cs[r * cs + (2 * pp + 1)];
      if (hh < p.Hq + p.Hkv) {
        const float2 rc = p.rope[(int64_t)t * half + i];  // (cos, sin) of t * theta^(-2i/Dh)
        const float a0 = y0 * rc.x - y1 * rc.y;
        const float a1 = y1 * rc.x + y0 * rc.y;
        y0 = a0;
        y1 = a1;
      }
      if (hh < p.Hq) {
        uint16_t *q = p.q_out + m * (int64_t)(p.Hq * p.Dh) + hh * p.Dh;
        q[i] = f2bf(y0);
        q[i + half] = f2bf(y1);
      } else {
        const bool isk = hh < p.Hq + p.Hkv;
        const int kvh = isk ? hh - p.Hq : hh - p.Hq - p.Hkv;
        uint16_t *dst = (isk ? p.k_cache : p.v_cache) +
                        (((int64_t)b * p.Hkv + kvh) * p.max_seq + t) * p.Dh;
        dst[i] = f2bf(y0);
        dst[i + half] = f2bf(y1);
      }
    }
  } else if constexpr (EP == kEpSwiGLU) {
    const int hw = BN / 2;
    for (int idx = tid; idx < BM * hw; idx += NTHR) {
      const int r = idx / hw, jj = idx % hw;
      const int64_t m = m0 + r;
      const int n = colblk * hw + jj;
      if (m >= p.M || n >= p.w.seg_rows[0]) continue;
      const float gt = Cs[r * cs + (jj)], up = Cs[r * cs + (hw + jj)];
      p.u_out[m * p.w.seg_rows[0] + n] = f2bf(gt / (1.0f + expf(-gt)) * up);
    }
  } else if constexpr (EP == kEpPlain) {
    for (int idx = tid; idx < BM * BN; idx += NTHR) {
      const int r = idx / BN, j = idx % BN;
      const int64_t m = m0 + r;
      const int n = colblk * BN + j;
      if (m < p.M && n < p.N) p.y_out[m * p.y_stride + n] = Cs[r * cs + (j)];
    }
  } else {  // residual
    for (int idx = tid; idx < BM * BN; idx += NTHR) {
      const int r = idx / BN, j = idx % BN;
      const int64_t m = m0 + r;
      const int n = colblk * BN + j;
      if (m >= p.M || n >= p.N) continue;
      const int64_t o = m * p.h_io_stride + n;
      p.h_out[o] = p.h_in[o] + Cs[r * cs + (j)];
    }
  }
}

// Prefill GEMMs of a layer at or past the exit under a comparator strategy:
// o passes the residual stream through, gate|up and down do nothing, q|k|v
// computes the k and v column blocks only, from the backbone weights (ex is
// set to false for them).  Returns true when the workgroup has nothing to do.
template <int EP, int BN>
__device__ __forceinline__ bool past_exit_skip(const GemmParams &p, int colblk, bool &ex) {
  if constexpr (EP != kEpQKV && EP != kEpResid && EP != kEpSwiGLU) return false;
  const int action = past_exit_action(p.ctrl, p.layer, p.path);
  if (action == kRun) return false;
  if constexpr (EP == kEpResid) {
    // the residual stream passes through (rows of earlier positions under the
    // recompute comparator: nothing is written back past the exit)
    if (p.path == kPathPending || p.h_out == p.h_in) return true;
    const int64_t nb = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    const int64_t i0 = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (int64_t idx = i0; idx < (int64_t)p.M * p.N; idx += nb) {
      const int64_t o = (idx / p.N) * p.h_io_stride + idx % p.N;
      p.h_out[o] = p.h_in[o];
    }
    return true;
  } else if constexpr (EP == kEpQKV) {
    if (action == kSkip) return true;
    ex = false;
    return (colblk + 1) * BN <= p.Hq * p.Dh;   // a block of query columns only
  } else {
    return true;
  }
}

template <int BM, int BN, int EP>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int LDSK = kBK + kLdsPad;
  constexpr int TM = BM / 32, TN = BN / 32;   // 16x16 tiles per wave
  __shared__ __align__(16) uint16_t As[BM][LDSK];
  __shared__ __align__(16) uint16_t Bs[BN][LDSK];
  __shared__ float Cs[BM][BN + 1];
  __shared__ uint32_t szs[BN];
  __shared__ float xsg[BM];

  bool ex = p.path == kPathDevice ? layer_uses_exit(p.ctrl, p.layer) : p.path == kPathExit;
  if (past_exit_skip<EP, BN>(p, blockIdx.y, ex)) return;   // (comparators)
  const bool q4 = ex && p.exit_mode == RIVER_EXIT_INT4;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.x * BM;
  const int KG = p.K / p.G;
  const int steps_per_group = p.G / kBK;

  // weight rows this thread loads (one tile row per thread when tid < BN)
  const uint16_t *brow = nullptr;
  const uint32_t *qrow = nullptr;
  const uint32_t *zrow = nullptr;
  bool bvalid = false;
  if (tid < BN) {
    int seg, row;
    map_col<EP>(p, blockIdx.y, BN, tid, seg, row, bvalid);
    if (!bvalid) row = 0;
    if (q4) {
      qrow = p.w.q4[seg] + (int64_t)row * (p.K / 8);
      zrow = p.w.sz[seg] + (int64_t)row * KG;
    } else {
      const uint16_t *bf = ex ? p.w.ex_bf[seg] : p.w.bf[seg];
      brow = bf + (int64_t)row * p.K;
    }
  }

  f32x4_t acc[TM][TN], tot[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) { acc[a][b][v] = 0.f; tot[a][b][v] = 0.f; }

  const int nsteps = p.K / kBK;
  for (int st = 0; st < nsteps; ++st) {
    const int k0 = st * kBK;
    // ---- stage A (BM x 32 bf16: 4 uint4 per row)
    for (int idx = tid; idx < BM * 4; idx += 256) {
      const int r = idx >> 2, c = idx & 3;
      const int64_t m = m0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < p.M) v = *reinterpret_cast<const uint4 *>(p.x + m * p.ldx + k0 + c * 8);
      *reinterpret_cast<uint4 *>(&As[r][c * 8]) = v;
    }
    // ---- stage B
    if (tid < BN) {
      if (q4) {
        uint4 cw = bvalid ? *reinterpret_cast<const uint4 *>(qrow + (k0 >> 3))
                          : make_uint4(0, 0, 0, 0);
        const uint32_t wd[4] = {cw.x, cw.y, cw.z, cw.w};
        // word i covers columns 8i..8i+7 (bf16 128+q in column order)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t o[4];
          unpack_word(wd[i], o);
          *reinterpret_cast<uint4 *>(&Bs[tid][i * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        if (st % steps_per_group == 0) szs[tid] = bvalid ? zrow[k0 / p.G] : 0u;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint4 v = bvalid ? *reinterpret_cast<const uint4 *>(brow + k0 + c * 8) : make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4 *>(&Bs[tid][c * 8]) = v;
        }
      }
    }
    __syncthreads();
    if (q4 && tid < BM) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kBK; ++c) s += bf2f(As[tid][c]);
      xsg[tid] = (st % steps_per_group == 0) ? s : xsg[tid] + s;
    }
    // ---- MFMA
    {
      bf16x8_t af[TM], bfr[TN];
      const int rr = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t *>(&As[wm * (BM / 2) + a * 16 + rr][kq]);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8_t *>(&Bs[wn * (BN / 2) + b * 16 + rr][kq]);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
    if (q4 && (st % steps_per_group) == steps_per_group - 1) {
      // fold the finished group: tot += s * (acc - (128 + z) * sum_k x)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int col = wn * (BN / 2) + b * 16 + (lane & 15);
          const uint32_t w = szs[col];
          const float s = bf_lo(w), zo = 128.0f + bf_hi(w);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wm * (BM / 2) + a * 16 + (lane >> 4) * 4 + v;
            tot[a][b][v] = fmaf(s, acc[a][b][v] - zo * xsg[row], tot[a][b][v]);
            acc[a][b][v] = 0.f;
          }
        }
      __syncthreads();
    }
  }

  // ---- results to LDS
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int col = wn * (BN / 2) + b * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * (BM / 2) + a * 16 + (lane >> 4) * 4 + v;
        Cs[row][col] = q4 ? tot[a][b][v] : acc[a][b][v];
      }
    }
  __syncthreads();

  tile_epilogue<EP, BN>(p, &Cs[0][0], BN + 1, BM, m0, blockIdx.y);
}

template <int EP>
static hipError_t gemm_launch_ep(const GemmParams &p, hipStream_t s) {
  constexpr int BM = 64, BN = 64;
  int ncols = p.N;
  if (EP == kEpSwiGLU) ncols = 2 * p.w.seg_rows[0];
  dim3 grid((p.M + BM - 1) / BM, (ncols + BN - 1) / BN);
  return launch_1(gemm_kernel<BM, BN, EP>, grid, dim3(256), p, s);
}

hipError_t launch_gemm(Epilogue ep, const GemmParams &p, hipStream_t s) {
  if (p.K % kBK || p.G % kBK) return hipErrorInvalidValue;
  switch (ep) {
    case kEpQKV: return gemm_launch_ep<kEpQKV>(p, s);
    case kEpSwiGLU: return gemm_launch_ep<kEpSwiGLU>(p, s);
    case kEpResid: return gemm_launch_ep<kEpResid>(p, s);
    case kEpPlain: return gemm_launch_ep<kEpPlain>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// ===========================================================================
// Causal GQA attention over the prompt (flash-style online softmax).
//   Workgroup (query block of 64 rows, q head, b); 4 threads per query row,
//   each owning Dh/4 of the head dimension; K/V tiles of 16 positions staged
//   in LDS.  Scores q.k / sqrt(Dh), fp32 softmax.
// ===========================================================================
template <int DH>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillParams p) {
  if (past_exit_action(p.ctrl, p.layer, p.path) != kRun) return;   // (comparators)
  constexpr int SL = DH / 4;    // elements per thread
  constexpr int KT = 16;        // keys per tile (measured: 16 beats 8, 32 and 64)
  __shared__ __align__(16) uint16_t Ks[KT][DH];
  __shared__ __align__(16) uint16_t Vs[KT][DH];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (p.Hq / p.Hkv);
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int t = qb * 64 + r;
  const bool live = t < p.T;
  const int64_t qrow = (int64_t)b * p.T + t;
  const int tpos = p.start + t;               // the query's position
  float q[SL], acc[SL];
#pragma unroll
  for (int e = 0; e < SL; ++e) { q[e] = 0.f; acc[e] = 0.f; }
  if (live) {
    const uint16_t *qp = p.q + qrow * (int64_t)(p.Hq * DH) + h * DH + part * SL;
#pragma unroll
    for (int e = 0; e < SL; e += 8) {
      const uint4 u = *reinterpret_cast<const uint4 *>(qp + e);
      q[e + 0] = bf_lo(u.x); q[e + 1] = bf_hi(u.x); q[e + 2] = bf_lo(u.y); q[e + 3] = bf_hi(u.y);
      q[e + 4] = bf_lo(u.z); q[e + 5] = bf_hi(u.z); q[e + 6] = bf_lo(u.w); q[e + 7] = bf_hi(u.w);
    }
  }
  float mrun = -INFINITY, lrun = 0.f;
  const int kend = p.start + min(p.T, qb * 64 + 64);  // keys needed by this block
  const int64_t kvbase = (((int64_t)b * p.Hkv + kvh) * p.S) * DH;
  for (int k0 = 0; k0 < kend; k0 += KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < KT * DH / 8; idx += 256) {
      const int kr = idx / (DH / 8), c = idx % (DH / 8);
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (k0 + kr < kend) {
        kv = *reinterpret_cast<const uint4 *>(p.k_cache + kvbase + (int64_t)(k0 + kr) * DH + c * 8);
        vv = *reinterpret_cast<const uint4 *>(p.v_cache + kvbase + (int64_t)(k0 + kr) * DH + c * 8);
      }
      *reinterpret_cast<uint4 *>(&Ks[kr][c * 8]) = kv;
      *reinterpret_cast<uint4 *>(&Vs[kr][c * 8]) = vv;
    }
    __syncthreads();
    float sc[KT];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < SL; ++e) d = fmaf(q[e], bf2f(Ks[j][part * SL + e]), d);
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      const bool ok = live && (k0 + j) <= tpos;
      sc[j] = ok ? d * p.scale : -INFINITY;
      tmax = fmaxf(tmax, sc[j]);
    }
    if (tmax == -INFINITY) continue;  // nothing visible in this tile (uniform per row)
    const float mnew = fmaxf(mrun, tmax);
    const float corr = expf(mrun - mnew);
    lrun *= corr;
#pragma unroll
    for (int e = 0; e < SL; ++e) acc[e] *= corr;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float pj = expf(sc[j] - mnew);
      lrun += pj;
#pragma unroll
      for (int e = 0; e < SL; ++e) acc[e] = fmaf(pj, bf2f(Vs[j][part * SL + e]), acc[e]);
    }
    mrun = mnew;
  }
  if (live) {
    uint16_t *op = p.out + qrow * (int64_t)(p.Hq * DH) + h * DH + part * SL;
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int e = 0; e < SL; e += 2) {
      *reinterpret_cast<uint32_t *>(op + e) = pack_bf2(acc[e] * inv, acc[e + 1] * inv);
    }
  }
}

// ===========================================================================
// Causal GQA attention over the prompt on the matrix cores (flash-style).
//   Workgroup: 64 query positions x GQ query heads of one kv head x row b;
//   wavefront w takes query positions q0 + 16 w .. +15 for all GQ heads, so
//   every K/V tile is loaded once for 4 * 16 * GQ query rows.  GQ is all the
//   kv head's query heads, or a half or a quarter of them when the grid would
//   otherwise hold fewer workgroups than CUs (short prompts of few rows).  Tiles of 32
//   key positions sit in LDS, double-buffered: K row-major with its 16-byte
//   chunks XOR-swizzled by the row, V transposed (V^T[dim][key]).
//   Scores as S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys x queries: each
//   lane then holds one query's scores, 4 keys of each 16-key half); online
//   softmax in fp32 in the base-2 domain; O^T = V^T P^T, with P split exactly
//   into three bf16 terms (p = p1 + p2 + p3, each the top 8 significant bits
//   of what is left), so the probabilities enter the products with all 24
//   bits and every sum is fp32.  The lanes' key order inside a k-step
//   ({4q..4q+3} and {16+4q..16+4q+3} for lane quarter q) is the same in the
//   A operand (V^T) and in the B operand (P^T), so the products pair up.
// ===========================================================================
template <int DH>
__device__ __forceinline__ int flash_swz(int r) {
  return DH == 128 ? (r & 15) : ((r >> 1) & 7);
}

constexpr float kLazyLog2 = 8.0f;   // largest probability taken against a stale maximum: 2^8

template <int DH, int GQ>
__global__ __launch_bounds__(256) void attn_flash_kernel(AttnPrefillParams p) {
  if (past_exit_action(p.ctrl, p.layer, p.path) != kRun) return;   // (comparators)
  constexpr int KT = 32;                // key positions per tile
  constexpr int CPR = DH / 8;           // 16-byte chunks per key row
  constexpr int NS = DH / 32;           // k-steps of a score MFMA
  constexpr int NO = DH / 16;           // output tiles of 16 dims
  constexpr int VST = KT + 4;           // V^T row stride (bf16): 72 bytes
  constexpr int NCH = KT * CPR / 256;   // 16-byte chunks per thread per tile
  __shared__ __align__(16) uint16_t Ks[2][KT * DH];
  __shared__ __align__(16) uint16_t Vt[2][DH * VST];

  const int qb = (int)gridDim.x - 1 - (int)blockIdx.x;   // longest rows first
  // blockIdx.y: GQ query heads from qh0 = GQ blockIdx.y on, all of kv head kvh
  const int kvh = (int)blockIdx.y / (p.Hq / (p.Hkv * GQ)), qh0 = (int)blockIdx.y * GQ, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c16 = lane & 15;
  const int q0 = qb * 64;
  const int my_q = q0 + 16 * wid + c16;         // this lane's query row
  const int qpos = p.start + my_q;              // and its position
  const int kall = p.start + p.T;               // key positions in the cache
  const int kend = p.start + min(p.T, q0 + 64); // key positions the workgroup needs
  const int ntiles = (kend + KT - 1) / KT;
  const int64_t kvbase = ((int64_t)b * p.Hkv + kvh) * p.S * DH;
  const uint16_t *Kg = p.k_cache + kvbase, *Vg = p.v_cache + kvbase;
  const float scale2 = p.scale * 1.4426950408889634f;

  // Q^T operands: lane (q, c16) holds dims 32 s + 8 q .. +7 of query my_q
  bf16x8_t qf[GQ][NS];
  {
    const int row = min(my_q, p.T - 1);
    const uint16_t *qp = p.q + ((int64_t)b * p.T + row) * (int64_t)(p.Hq * DH) + (int64_t)qh0 * DH + 8 * q;
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int st = 0; st < NS; ++st)
        qf[h][st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qp + h * DH + 32 * st));
  }

  // one tile: thread tid moves 16-byte chunks tid + 256 u of K and of V
  uint4 kr[NCH], vr[NCH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int ch = tid + 256 * u, r = ch / CPR, cc = ch % CPR;
      const int pos = min(kt * KT + r, kall - 1);  // past the last key: masked below
      kr[u] = *reinterpret_cast<const uint4 *>(Kg + (int64_t)pos * DH + 8 * cc);
      vr[u] = *reinterpret_cast<const uint4 *>(Vg + (int64_t)pos * DH + 8 * cc);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int ch = tid + 256 * u, r = ch / CPR, cc = ch % CPR;
      *reinterpret_cast<uint4 *>(&Ks[buf][(r * CPR + (cc ^ flash_swz<DH>(r))) * 8]) = kr[u];
      const uint32_t w4[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[buf][(8 * cc + 2 * e) * VST + r] = (uint16_t)(w4[e] & 0xFFFFu);
        Vt[buf][(8 * cc + 2 * e + 1) * VST + r] = (uint16_t)(w4[e] >> 16);
      }
    }
  };

  float m[GQ], lsum[GQ];
  f32x4_t o[GQ][NO];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < NO; ++j) o[h][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);   // in flight while this tile is reduced
    const uint16_t *K = Ks[buf];
    const uint16_t *V = Vt[buf];
    // K operands of both 16-key halves: lane (q, c16) = key 16 kk + c16, dims 32 s + 8 q
    bf16x8_t ka[2][NS];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r = 16 * kk + c16;
#pragma unroll
      for (int st = 0; st < NS; ++st)
        ka[kk][st] = *reinterpret_cast<const bf16x8_t *>(&K[(r * CPR + ((4 * st + q) ^ flash_swz<DH>(r))) * 8]);
    }
    // scores, online softmax and the three-term split of P, per head
    uint32_t pt[GQ][3][4];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int st = 0; st < NS; ++st)
          sc[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk][st], qf[h][st], sc[kk], 0, 0, 0);
      // this lane: query my_q against keys kt KT + 16 kk + 4 q + i
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt * KT + 16 * kk + 4 * q + i;
          const bool ok = key <= qpos && key < kall;
          sv[4 * kk + i] = ok ? sc[kk][i] * scale2 : -INFINITY;
          mx = fmaxf(mx, sv[4 * kk + i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // lazy rescaling: the reference maximum moves only when a score
      // exceeds it by more than 2^kLazyLog2; below that the probabilities are
      // taken against the old reference (at most 2^kLazyLog2, exact in fp32,
      // and the same reference divides out of O and the row sum), so the
      // output tiles are rescaled only in the rare tiles where some lane's
      // reference moved (the four lanes of a query agree: mx is their common
      // maximum)
      const bool bump = mx > m[h] + kLazyLog2;
      const float mref = bump ? mx : m[h];
      const float corr = bump ? exp2_fast(m[h] - mx) : 1.f;
      float part = 0.f;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
      if (mref != -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = exp2_fast(sv[e] - mref);
          part += pv[e];
        }
      }
      lsum[h] = lsum[h] * corr + part;   // this lane's share of the row sum
      m[h] = mref;
      if (__any(bump)) {
#pragma unroll
        for (int j = 0; j < NO; ++j) o[h][j] *= corr;
      }
      // p = p1 + p2 + p3 exactly: each term keeps the top 16 bits of what is
      // left (a bf16 value), the subtractions are exact
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t t1[2], t2[2], t3[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const float v = pv[2 * e + x];
          const float v1 = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
          const float r1 = v - v1;
          const float v2 = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
          const float v3 = r1 - v2;          // has at most 8 significant bits: a bf16 value
          t1[x] = __float_as_uint(v1);
          t2[x] = __float_as_uint(v2);
          t3[x] = __float_as_uint(v3);
        }
        pt[h][0][e] = __builtin_amdgcn_perm(t1[1], t1[0], 0x07060302u);
        pt[h][1][e] = __builtin_amdgcn_perm(t2[1], t2[0], 0x07060302u);
        pt[h][2][e] = __builtin_amdgcn_perm(t3[1], t3[0], 0x07060302u);
      }
    }
    // O^T += V^T P^T: lane (q, c16) reads dim 16 j + c16 at keys {4q..4q+3} and {16+4q..16+4q+3}
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const uint16_t *vrow = V + (16 * j + c16) * VST + 4 * q;
      const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16);
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
      for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int t = 0; t < 3; ++t)
          o[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              va, __builtin_bit_cast(bf16x8_t, make_uint4(pt[h][t][0], pt[h][t][1], pt[h][t][2], pt[h][t][3])),
              o[h][j], 0, 0, 0);
    }
    if (kt + 1 < ntiles) {
      // the other buffer was last read in the previous iteration, which every
      // wavefront finished before the barrier that ended it
      lstore((kt + 1) & 1);
      __syncthreads();
    }
  }

  // row sums over the four lane quarters; O^T lane (q, c16): dims 16 j + 4 q + i of query my_q
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float lt = lsum[h];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = 1.0f / lt;
    if (my_q < p.T) {
      uint16_t *op = p.out + ((int64_t)b * p.T + my_q) * (int64_t)(p.Hq * DH) + ((int64_t)qh0 + h) * DH + 4 * q;
#pragma unroll
      for (int j = 0; j < NO; ++j) {
        const f32x4_t v = o[h][j];
        *reinterpret_cast<uint2 *>(op + 16 * j) =
            make_uint2(pack_bf2(v[0] * inv, v[1] * inv), pack_bf2(v[2] * inv, v[3] * inv));
      }
    }
  }
}

// Query heads per workgroup: all of a kv head's, halved while the grid would
// hold fewer workgroups than CUs (256 on this chip); each split loads the kv
// head's K/V tiles itself (from L2).  At one 512-token prompt of the 8B shape
// (64 workgroups with all four heads, 256 with one) the attention 67 -> 34 us
// per layer, the prefill 26.2K -> 27.6K tokens/s.
template <int DH>
static hipError_t attn_flash_launch(const AttnPrefillParams &p, hipStream_t s) {
  const int g = p.Hq / p.Hkv, nqb = (p.T + 63) / 64;
  if (g != 1 && g != 2 && g != 4) return hipErrorInvalidValue;
  int gq = g;
  while (gq > 1 && (int64_t)nqb * p.Hkv * (g / gq) * p.B < 256) gq /= 2;
  dim3 grid(nqb, p.Hkv * (g / gq), p.B);
  switch (gq) {
    case 1: return launch_1(attn_flash_kernel<DH, 1>, grid, dim3(256), p, s);
    case 2: return launch_1(attn_flash_kernel<DH, 2>, grid, dim3(256), p, s);
    case 4: return launch_1(attn_flash_kernel<DH, 4>, grid, dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_prefill(const AttnPrefillParams &p, hipStream_t s) {
  if (p.mfma) {
    switch (p.Dh) {
      case 64: return attn_flash_launch<64>(p, s);
      case 128: return attn_flash_launch<128>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  dim3 grid((p.T + 63) / 64, p.Hq, p.B);
  switch (p.Dh) {
    case 64: return launch_1(attn_prefill_kernel<64>, grid, dim3(256), p, s);
    case 128: return launch_1(attn_prefill_kernel<128>, grid, dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}


// ===========================================================================
// Prefill GEMM for many rows: Y[m][n] = sum_k X[m][k] W[n][k] on
// v_mfma_f32_16x16x32_bf16.  Workgroup tile 128 rows x BN columns, eight
// wavefronts of 64 columns each: BN = 128 as 4 x 2 wavefronts of 32 x 64, BN
// = 256 (from 4,096 rows) as 2 x 4 of 64 x 64, where every B operand feeds
// four MFMAs instead of two; two wavefronts per SIMD so that one's waits
// overlap the other's MFMAs.
//   Every operand goes straight from memory into LDS (global_load_lds, no
//   registers), three k-tile buffers, so two tiles are in flight while one
//   feeds the MFMAs.  Rows (and bf16 weight rows) are stored whole, their
//   16-byte chunks XOR-swizzled (chunk c of row r at slot r * CH + (c ^ (r mod
//   CH)), CH chunks per row), so that one copy instruction reads whole rows
//   from memory.  A 16-byte LDS read runs at the full rate only when each
//   quarter wavefront (16 lanes) reads one contiguous 256-byte block; the
//   fragment reads here (16 rows at one chunk) take about 1.45x that, but a
//   layout with conflict-free fragment reads needs copies of 64 bytes per row
//   and measured slower overall (int4 -8%, bf16 -20%).
//   int4 weights: k-tiles of 128; the codes of 16 columns stored as 4 blocks
//   of (one quarter's 4 words of each column), so that each quarter of a code
//   read is one 256-byte block; the scale/zero words beside them (per-group
//   accumulation, lane quarters over G/4 codes, group fold
//   tot += s * (acc - (128 + z) * sum_k x), the row sums of each group from
//   one more MFMA per row block against a B operand of ones).
//   bf16 weights: k-tiles of 64 (rows and weights of three tiles then fit
//   the same LDS).
//   Workgroups are ordered in groups of 32 row blocks so that the weights
//   they share stay in L2 (against 8: bf16 weights +13%, int4 +1.5% at 32K
//   rows).
// ===========================================================================
constexpr int kPBM = 128, kPGroupRows = 32;
constexpr int kPThreads = 512, kPBufs = 3;
constexpr int kPWideRows = 4096;                  // rows from which column blocks are 256 wide
// k-tile: 128 columns for int4 weights, 64 for bf16 weights
template <bool Q4> constexpr int pkt() { return Q4 ? 128 : 64; }
// 16-byte slots of BM rows per k-tile
template <bool Q4, int BM> constexpr int prow_slots() { return BM * pkt<Q4>() / 8; }
// 16-byte slots of weights per k-tile of BN columns (int4 codes or bf16)
template <bool Q4, int BN> constexpr int pw_slots() { return Q4 ? BN * pkt<Q4>() / 32 : BN * pkt<Q4>() / 8; }
// wavefronts along N (each 64 columns wide) and along M, rows per wavefront
// (NTH threads, BM rows per workgroup)
template <int BN> constexpr int pwn() { return BN / 64; }
template <int BN, int NTH = kPThreads> constexpr int pwm() { return NTH / 64 / pwn<BN>(); }
template <int BN, int NTH = kPThreads, int BM = kPBM> constexpr int ptm() { return BM / pwm<BN, NTH>(); }
// int4 scale/zero words per k-tile: one for each thread, or one for each
// (group, column) of the tile when there are more of those
template <int G, int BN, int NTH> constexpr int psz_words() {
  return NTH > (pkt<true>() / G) * BN ? NTH : (pkt<true>() / G) * BN;
}
// LDS of a workgroup: row buffers, weight buffers, scale/zero buffers (the
// results reuse them all)
template <bool Q4, int G, int BN, int NTH, int BM> constexpr int pstage_slots() {
  return prow_slots<Q4, BM>() + pw_slots<Q4, BN>() + (Q4 ? psz_words<G, BN, NTH>() / 4 : 0);
}
template <int G, int BN, int NTH = kPThreads, int BM = kPBM> constexpr int psmem_slots() {
  return kPBufs * (pstage_slots<true, G, BN, NTH, BM>() > pstage_slots<false, G, BN, NTH, BM>()
                       ? pstage_slots<true, G, BN, NTH, BM>()
                       : pstage_slots<false, G, BN, NTH, BM>());
}


// NTH threads take a BM x BN tile over the k-tiles kt0 .. kt0 + ntile - 1
// (k-tiles of this weight form); with C128 the columns are mapped as 128-column
// blocks (block colblk * BN / 128 + c / 128, column c mod 128), the layout of
// the batched-row GEMM's partial tiles.
template <int G, int EP, bool Q4, int BN, int NTH = kPThreads, int BM = kPBM, bool C128 = false>
__device__ __forceinline__ void pgemm_body(const GemmParams &p, uint4 *smem, bool ex, int rowblk, int colblk,
                                           int kt0, int ntile, f32x4_t (&tot)[ptm<BN, NTH, BM>() / 16][4]) {
  constexpr int KT = pkt<Q4>(), CH = KT / 8;               // k columns and 16-byte chunks per row
  constexpr int ASL = prow_slots<Q4, BM>(), WSL = pw_slots<Q4, BN>();
  constexpr int NA = ASL / NTH;                            // row copies per wavefront per k-tile
  constexpr int NW = WSL / NTH;                            // weight copies per wavefront per k-tile
  static_assert(ASL % NTH == 0 && WSL % NTH == 0, "whole copies");
  constexpr int SZW = psz_words<G, BN, NTH>(), NZ = Q4 ? SZW / NTH : 0;   // scale/zero copies
  constexpr int STEPS = G / 32, GW = G / 32;
  constexpr int NWAV = NTH / 64, WN = pwn<BN>(), TM = ptm<BN, NTH, BM>(), AF = TM / 16;
  static_assert(TM % 16 == 0 && pwm<BN, NTH>() * WN * 64 == NTH, "wavefront grid");
  uint4 *xs = smem, *ws = smem + kPBufs * ASL, *zs = ws + kPBufs * WSL;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, cl = lane & 15;
  const int wm = wid / WN, wn = wid % WN;
  const int64_t m0 = (int64_t)rowblk * BM;
  const int KG = p.K / G;
  auto col_of = [&](int c, int &seg, int &row, bool &valid) {
    if constexpr (C128) map_col<EP>(p, colblk * (BN / 128) + c / 128, 128, c % 128, seg, row, valid);
    else map_col<EP>(p, colblk, BN, c, seg, row, valid);
  };

  // ---- weights of a k-tile, copy i of this wavefront covers slots
  //      s = (NWAV i + wid) * 64 + lane (NWAV wavefronts).  int4: column c's quarter q (its words
  //      4q..4q+3) at slot ((c / 16) * 4 + q) * 16 + c % 16; bf16: chunk q
  //      of column n at slot n * CH + (q ^ (n mod CH))
  const void *wsrc[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int s = (i * NWAV + wid) * 64 + lane;
    int c, q;
    if constexpr (Q4) { c = (s >> 6) * 16 + (s & 15); q = (s >> 4) & 3; }
    else { c = s / CH; q = (s % CH) ^ (c & (CH - 1)); }
    int seg, row;
    bool valid;
    col_of(c, seg, row, valid);
    if (!valid) { seg = 0; row = 0; }
    // the segment is picked by selects, not by indexing the parameter arrays
    // with a per-lane value (that would copy them to scratch memory)
    if constexpr (Q4) {
      const uint32_t *b = seg == 0 ? p.w.q4[0] : seg == 1 ? p.w.q4[1] : p.w.q4[2];
      wsrc[i] = b + (int64_t)row * (p.K / 8) + 4 * q;
    } else {
      const uint16_t *b0 = ex ? p.w.ex_bf[0] : p.w.bf[0], *b1 = ex ? p.w.ex_bf[1] : p.w.bf[1],
                     *b2 = ex ? p.w.ex_bf[2] : p.w.bf[2];
      const uint16_t *b = seg == 0 ? b0 : seg == 1 ? b1 : b2;
      wsrc[i] = b + (int64_t)row * p.K + 8 * q;
    }
  }
  // ---- int4 scale/zero words: entry e = NTH z + 64 wid + lane of a k-tile
  //      is group e / BN of the k-tile for column e % BN (entries past the
  //      tile's groups repeat the last group)
  constexpr int GPT = KT / G;                   // groups per k-tile
  const uint32_t *zrow[NZ > 0 ? NZ : 1];
#pragma unroll
  for (int z = 0; z < NZ; ++z) {
    const int e = z * NTH + wid * 64 + lane;
    const int gi = min(e / BN, GPT - 1), c = e % BN;
    int seg, row;
    bool valid;
    col_of(c, seg, row, valid);
    if (!valid) { seg = 0; row = 0; }
    const uint32_t *b = seg == 0 ? p.w.sz[0] : seg == 1 ? p.w.sz[1] : p.w.sz[2];
    zrow[z] = b + (int64_t)row * KG + gi;
  }

  // ---- rows: copy i of this wavefront covers slots s = (wid * NA + i) * 64 +
  //      lane, i.e. row s / CH, chunk (s mod CH) ^ (row mod CH)
  const uint16_t *arow[NA];
  int acol[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int s = (wid * NA + i) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ (r & (CH - 1));
    const int64_t m = min(m0 + r, (int64_t)p.M - 1);      // rows past M: any valid row
    arow[i] = p.x + m * p.ldx;
    acol[i] = 8 * c;
  }
  // The copies are issued from inline assembly: the compiler then does not
  // treat every later LDS read as possibly overlapping them (it would wait for
  // all memory operations before each one); the loop waits for exactly the
  // copies it needs with an explicit s_waitcnt.  m0 holds the LDS destination
  // of a copy (each lane writes 16 bytes at m0 + 16 * lane).
  const uint32_t xs_base = (uint32_t)(uintptr_t)(lds_ptr_t)xs;
  const uint32_t ws_base = (uint32_t)(uintptr_t)(lds_ptr_t)ws;
  const uint32_t zs_base = (uint32_t)(uintptr_t)(lds_ptr_t)zs;
  const int uwid = __builtin_amdgcn_readfirstlane(wid);
  auto load_tile = [&](int kt) {
    const int ktc = kt0 + min(kt, ntile - 1);              // unconditional: fixed load count
    const int buf = kt % kPBufs;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(xs_base + (uint32_t)((buf * ASL + (uwid * NA + i) * 64) * 16));
      const uint16_t *src = arow[i] + ktc * KT + acol[i];
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src)
                   : "memory", "m0");
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(ws_base + (uint32_t)((buf * WSL + (i * NWAV + uwid) * 64) * 16));
      const void *src;
      if constexpr (Q4) src = static_cast<const uint32_t *>(wsrc[i]) + ktc * (KT / 8);
      else src = static_cast<const uint16_t *>(wsrc[i]) + ktc * KT;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src)
                   : "memory", "m0");
    }
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
      // scale/zero words: each lane writes 4 bytes at m0 + 4 * lane
      const uint32_t zdst =
          __builtin_amdgcn_readfirstlane(zs_base + (uint32_t)(buf * SZW * 4 + (z * NTH + uwid * 64) * 4));
      const uint32_t *zsrc = zrow[z] + ktc * GPT;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(zdst), "v"(zsrc)
                   : "memory", "m0");
    }
  };
  // row fragment: row 16 (wm * AF + a) + cl, chunk c of the k-tile
  auto a_frag = [&](const uint4 *buf, int a, int c) -> bf16x8_t {
    return __builtin_bit_cast(bf16x8_t, buf[((wm * AF + a) * 16 + cl) * CH + (c ^ (cl & (CH - 1)))]);
  };

  // int4: raw sums of a group (against the codes as 128+q per column tile,
  // and the row sums against ones) and its scale/zero words; each group is
  // folded right after its MFMAs (folding the second wavefront of each SIMD
  // one k-tile later, beside the other's MFMAs, measured 2.5% slower at 32K
  // rows with the current layouts)
  f32x4_t ag[AF][4], as[AF];
  uint32_t pz[4];
#pragma unroll
  for (int a = 0; a < AF; ++a) {
    as[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) ag[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // the group's fold: tot += s * (acc - (128 + z) * sum_k x)
  auto fold = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float sc = bf_lo(pz[t]), zo = 128.0f + bf_hi(pz[t]);
#pragma unroll
      for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) tot[a][t][v] = fmaf(sc, ag[a][t][v] - zo * as[a][v], tot[a][t][v]);
    }
  };

  // one group of G columns of int4 weights (kl: its first column in the k-tile)
  auto group_q4 = [&](int buf, int kl) {
    const uint4 *xb = xs + buf * ASL;
    // this lane's code words of the group, for each of its 4 column tiles:
    // word j of column tile t at cb[cslot[t] + j] (read per step, so that no
    // register array is indexed by the step)
    const uint32_t *cb = reinterpret_cast<const uint32_t *>(ws + buf * WSL);
    const int wo = (kl / G) * (G / 8) + qq * GW;        // first word within the column's 16
    int cslot[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) cslot[t] = (((wn * 4 + t) * 4 + (wo >> 2)) * 16 + cl) * 4 + (wo & 3);
    // the group sums of the rows come from one more MFMA per row block
    // against a B operand of ones (row sums in every column)
    const bf16x8_t ones =
        __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    // one k-step of 32: the row fragments (lane quarter qq takes chunk
    // (kl + qq G/4) / 8 + j), then one column tile at a time (its unpacked
    // operand feeds the AF MFMAs of the step and is dead after them); the
    // first step of a group starts its sums from zero
    auto kstep = [&](int j, bool first) {
      bf16x8_t af[AF];
#pragma unroll
      for (int a = 0; a < AF; ++a) af[a] = a_frag(xb, a, kl / 8 + qq * (G / 32) + j);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t pr[4];
        unpack_word(cb[cslot[t] + j], pr);
        const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, make_uint4(pr[0], pr[1], pr[2], pr[3]));
#pragma unroll
        for (int a = 0; a < AF; ++a)
          ag[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr, first ? zero4 : ag[a][t], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < AF; ++a)
        as[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], ones, first ? zero4 : as[a], 0, 0, 0);
    };
    kstep(0, true);
#pragma unroll
    for (int j = 1; j < STEPS; ++j) kstep(j, false);
    // this group's scale/zero words (read now: the buffer is refilled
    // after the next barrier)
    const uint32_t *zb = reinterpret_cast<const uint32_t *>(zs) + buf * SZW + (kl / G) * BN + wn * 64 + cl;
#pragma unroll
    for (int t = 0; t < 4; ++t) pz[t] = zb[t * 16];
    fold();
  };

  // a k-tile of bf16 weights: two k-steps of 32 in the natural order (lane
  // quarter qq takes chunk 4 j + qq)
  auto tile_bf16 = [&](int buf) {
    const uint4 *xb = xs + buf * ASL, *wb = ws + buf * WSL;
#pragma unroll
    for (int j = 0; j < KT / 32; ++j) {
      bf16x8_t af[AF];
#pragma unroll
      for (int a = 0; a < AF; ++a) af[a] = a_frag(xb, a, 4 * j + qq);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sl = ((wn * 4 + t) * 16 + cl) * CH + ((4 * j + qq) ^ (cl & (CH - 1)));
        const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, wb[sl]);
#pragma unroll
        for (int a = 0; a < AF; ++a)
          tot[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr, tot[a][t], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < kPBufs - 1; ++t) load_tile(t);
  for (int kt = 0; kt < ntile; ++kt) {
    // tile kt has landed once no more than the copies of the next
    // kPBufs - 2 k-tiles are outstanding (every copy is unconditional, so the
    // count holds throughout)
    constexpr int per_tile = NA + NW + NZ;
    constexpr int later = (kPBufs - 2) * per_tile;
    static_assert(later < 64, "vmcnt field");
    // s_waitcnt: vmcnt = later, expcnt and lgkmcnt not waited for
    __builtin_amdgcn_s_waitcnt((later & 0xF) | (0x7 << 4) | (0xF << 8) | ((later >> 4) << 14));
    __syncthreads();                        // tile kt visible; tile kt-1 done everywhere
    load_tile(kt + kPBufs - 1);             // into the buffer tile kt-1 used
    const int buf = kt % kPBufs;
    if constexpr (Q4) {
#pragma unroll
      for (int g = 0; g < GPT; ++g) group_q4(buf, g * G);
    } else {
      tile_bf16(buf);
    }
  }
  // the last k-tiles' spare copies may still be landing in LDS, which the
  // results reuse: wait for every memory operation, then for every wavefront
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// ===========================================================================
// Batched-row GEMM for 9..64 rows: Y[m][n] = sum_k X[m][k] W[n][k].
//   A workgroup (4 wavefronts x 2 column tiles of 16 = 128 columns) takes one
//   split of K.  Every lane loads the weights of its own output column straight
//   from HBM into MFMA B operands, several quantisation groups ahead of use;
//   the rows X of the whole split sit in LDS.  K is walked one group (G
//   columns) at a time.  int4: lane quarter qq holds the G/4 codes
//   k0 + qq*G/4 .. (unpacked in column order by the byte permute), so every
//   MFMA sums inside one group, which is then folded as
//   tot += s * (acc - (128 + z) * sum_k x).
//   bf16 weights use the plain order (quarter qq holds k0 + 32j + 8qq .. +8).
//   With several K splits each workgroup stores its partial tile and a second
//   kernel (one workgroup per column block) adds the splits in order and runs
//   the epilogue.
// ===========================================================================

// LM head argmax key of logit v in column n: value order, then lowest index
__device__ __forceinline__ uint64_t logit_key(float v, int n) {
  return ((uint64_t)float_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)n);
}

// End of an LM head workgroup: its per-row keys (rows m0 .. m0 + ROWS, in
// LDS, complete) go to the launch-wide maxima, and the last workgroup of the
// launch writes the next tokens and the pass bookkeeping (E histogram,
// position).
template <int ROWS>
__device__ void logits_finish(const GemmParams &p, int m0, uint64_t *rowkey, int *last_flag) {
  Control *ctl = p.ctrl;
  if (threadIdx.x < ROWS && m0 + (int)threadIdx.x < p.M)
    __hip_atomic_fetch_max(control_keys(ctl) + m0 + threadIdx.x, rowkey[threadIdx.x], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  if (arrive_last(&ctl->counters[kCtrLogits], gridDim.x, last_flag)) {
    if (threadIdx.x < p.M && p.next) {
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

// LM head epilogue of one column block: logits out, per-row argmax keys, then
// logits_finish.
template <int ROWS, int BN>
__device__ void logits_epilogue(const GemmParams &p, const float *Cs, int m0, int colblk,
                                uint64_t *rowkey, int *last_flag) {
  if (threadIdx.x < ROWS) rowkey[threadIdx.x] = 0;
  __syncthreads();
  for (int idx = threadIdx.x; idx < ROWS * BN; idx += 256) {
    const int r = idx / BN, j = idx % BN;
    const int n = colblk * BN + j;
    if (m0 + r >= p.M || n >= p.N) continue;
    const float v = Cs[r * (BN + 1) + j];
    if (p.logits) p.logits[(int64_t)(m0 + r) * p.vocab + n] = v;
    __hip_atomic_fetch_max(&rowkey[r], logit_key(v, n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  logits_finish<ROWS>(p, m0, rowkey, last_flag);
}

template <int MB, int G> struct MgemmShape {
  static constexpr int NT = 2;                    // column tiles per wavefront
  static constexpr int BN = kMgemmBN;             // 4 x NT x 16
  static constexpr int ROWS = MB * 16;
  // K columns of the rows held in LDS: the whole K split of a workgroup is
  // staged once, before any weight load is issued, so the weight stream never
  // waits behind activation loads (about 66 KB: two workgroups per CU)
  static constexpr int KS = MB == 1 ? 2048 : MB == 2 ? 1024 : 512;
  static constexpr int XS = KS + 8;               // padded LDS row (bf16)
  static constexpr int STEPS = G / 32;            // MFMA k-steps per group
  static constexpr int GW = G / 32;               // code words per lane per group
  static constexpr int XBYTES = ROWS * XS * 2;
  static constexpr int CBYTES = ROWS * (BN + 1) * 4;
  static constexpr int SMEM = XBYTES > CBYTES ? XBYTES : CBYTES;
  static_assert(KS % G == 0, "slab holds whole groups");
};

struct MgemmLds {
  uint16_t *xs;        // staged rows [ROWS][XS]
  float *xsg;          // [ROWS][KS/G] group sums of the staged rows (int4)
};

// Main loop of the batched-row GEMM over this workgroup's K split, for one
// weight form (Q4: int4 exit copy; else bf16).  Weights run D groups ahead.
template <int MB, int G, int EP, bool Q4>
__device__ __forceinline__ void mgemm_body(const GemmParams &p, const MgemmLds &L, bool ex, int colblk,
                                           int kbeg, int kend,
                                           f32x4_t (&tot)[MB][MgemmShape<MB, G>::NT]) {
  typedef MgemmShape<MB, G> S;
  constexpr int NT = S::NT, BN = S::BN, ROWS = S::ROWS, KS = S::KS, XS = S::XS;
  constexpr int STEPS = S::STEPS, GW = S::GW;
  // groups in flight per lane: two (measured at 16 and 32 rows: deeper
  // look-ahead makes the row staging, which waits for every load issued
  // before it, start later, and saves no latency once the loop runs)
  constexpr int D = 2;
  typedef typename WordsT<GW>::T WT;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, cl = lane & 15;
  const int nchunk = (kend - kbeg) / G;
  const int KG = p.K / G;

  const uint16_t *brow[NT];
  const uint32_t *qrow[NT], *zrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int seg, row;
    bool valid;
    map_col<EP>(p, colblk, BN, wid * (NT * 16) + t * 16 + cl, seg, row, valid);
    if (!valid) { seg = 0; row = 0; }      // a valid row; its results are dropped
    // segments picked by selects (a per-lane index into the parameter arrays
    // would copy them to scratch memory)
    if constexpr (Q4) {
      qrow[t] = (seg == 0 ? p.w.q4[0] : seg == 1 ? p.w.q4[1] : p.w.q4[2]) + (int64_t)row * (p.K / 8);
      zrow[t] = (seg == 0 ? p.w.sz[0] : seg == 1 ? p.w.sz[1] : p.w.sz[2]) + (int64_t)row * KG;
    } else {
      const uint16_t *b0 = ex ? p.w.ex_bf[0] : p.w.bf[0], *b1 = ex ? p.w.ex_bf[1] : p.w.bf[1],
                     *b2 = ex ? p.w.ex_bf[2] : p.w.bf[2];
      brow[t] = (seg == 0 ? b0 : seg == 1 ? b1 : b2) + (int64_t)row * p.K;
    }
  }

  WT wq[D][NT];
  uint32_t wz[D][NT];
  v4u wb[D][NT][STEPS];
  auto load = [&](int c, int u) {
    const int k0 = kbeg + c * G;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (Q4) {
        wq[u][t] = __builtin_nontemporal_load(
            reinterpret_cast<const WT *>(qrow[t] + (k0 >> 3) + qq * GW));
        wz[u][t] = zrow[t][k0 / G];
      } else {
#pragma unroll
        for (int j = 0; j < STEPS; ++j)
          wb[u][t][j] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u *>(brow[t] + k0 + 32 * j + 8 * qq));
      }
    }
  };

  const int slab0 = kbeg;
  // the rows of the split: all their loads are issued first, before any
  // weight load, so that waiting for them does not wait for the weights (a
  // wait counts loads in issue order); they land in LDS with their group sums
  // once the first weight groups are in flight too
  constexpr int PER = ROWS * (KS / 8) / 256;      // items per thread at most
  uint4 xv[PER];
  auto stage_load = [&](int base) {
    const int n8 = (kend - base) >> 3;
    const int total = ROWS * n8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int m = idx / n8, g8 = idx - m * n8;
      xv[i] = make_uint4(0, 0, 0, 0);
      if (idx < total && m < p.M)
        xv[i] = *reinterpret_cast<const uint4 *>(p.x + (int64_t)m * p.ldx + base + 8 * g8);
    }
  };
  auto stage_store = [&](int base) {
    const int n8 = (kend - base) >> 3;
    const int total = ROWS * n8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < total) {
        const int m = idx / n8, g8 = idx - m * n8;
        const uint4 w = xv[i];
        if constexpr (Q4) {
          // group sum: the G/8 items of a group sit in G/8 adjacent lanes
          // (n8 and the 256-thread stride are multiples of G/8)
          float gs = ((bf_lo(w.x) + bf_hi(w.x)) + (bf_lo(w.y) + bf_hi(w.y))) +
                     ((bf_lo(w.z) + bf_hi(w.z)) + (bf_lo(w.w) + bf_hi(w.w)));
          gs = G == 128 ? sum16(gs) : sum8(gs);
          if (g8 % (G / 8) == 0) L.xsg[m * (KS / G) + g8 / (G / 8)] = gs;
        }
        *reinterpret_cast<uint4 *>(L.xs + m * XS + 8 * g8) = w;
      }
    }
    __syncthreads();
  };

  auto compute = [&](int c, int u) {
    const int kl = kbeg + c * G - slab0;
    if constexpr (Q4) {
      f32x4_t ag[MB][NT];
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int t = 0; t < NT; ++t) ag[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        bf16x8_t af[MB], bfr[NT];
#pragma unroll
        for (int a = 0; a < MB; ++a)
          af[a] = *reinterpret_cast<const bf16x8_t *>(L.xs + (a * 16 + cl) * XS + kl + qq * (G / 4) + 8 * j);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint32_t w;
          if constexpr (GW == 1) w = wq[u][t];
          else w = wq[u][t][j];
          uint32_t pr[4];
          unpack_word(w, pr);
          bfr[t] = __builtin_bit_cast(bf16x8_t, make_uint4(pr[0], pr[1], pr[2], pr[3]));
        }
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            ag[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[t], ag[a][t], 0, 0, 0);
      }
      const int g = kl / G;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float sc = bf_lo(wz[u][t]), zo = 128.0f + bf_hi(wz[u][t]);
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            tot[a][t][v] = fmaf(sc, ag[a][t][v] - zo * L.xsg[(a * 16 + 4 * qq + v) * (KS / G) + g],
                                tot[a][t][v]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        bf16x8_t af[MB];
#pragma unroll
        for (int a = 0; a < MB; ++a)
          af[a] = *reinterpret_cast<const bf16x8_t *>(L.xs + (a * 16 + cl) * XS + kl + 32 * j + 8 * qq);
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            tot[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                af[a], __builtin_bit_cast(bf16x8_t, wb[u][t][j]), tot[a][t], 0, 0, 0);
      }
    }
  };

  // the rows of the whole split (the plan keeps it within KS), then the first
  // D groups of weights, so both latencies overlap; after that the loop only
  // ever waits for the oldest weight group
  stage_load(kbeg);
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < nchunk) load(u, u);
  stage_store(kbeg);
  for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int c = c0 + u;
      if (c < nchunk) {
        compute(c, u);
        if (c + D < nchunk) load(c + D, u);
      }
    }
  }
}

// int4 layers through the copy ring (p.ring = RBN, the column block): RBN =
// 256 or 128 columns of the rows (ROWS = 16 MB of them) over one K split, on
// the prefill GEMM's body with 256 threads (4 wavefronts of 64 columns: 1 x 4,
// or 2 x 2 for 128-column blocks of 32 or more rows); rows, codes and
// scale/zero words reach LDS by DMA, three k-tiles deep.  The partial tile
// goes out in the 128-column layout that the reduce kernel adds (the plan
// always splits K).  The LM head (bf16 weights, Q4 false) takes the same ring
// from 17 rows on: every k-tile then reads whole 128-byte lines of 256 weight
// rows, where the register path reads each row in 64-byte pieces.
template <int MB> constexpr int mgemm_ring_bm() { return MB * 16; }
template <int MB, int G, bool Q4 = true, int RBN = 256> constexpr int mgemm_ring_bytes() {
  return kPBufs * pstage_slots<Q4, G, RBN, 256, mgemm_ring_bm<MB>()>() * 16;
}
constexpr int kLogitsRbn = 128;   // column block of the LM head's ring

template <int MB, int G, int EP, int RBN, bool Q4 = true>
__device__ void mgemm_ring(const GemmParams &p, uint4 *smem, bool ex) {
  constexpr int BM = mgemm_ring_bm<MB>(), WN = RBN / 64, TM = ptm<RBN, 256, BM>(), AF = TM / 16;
  static_assert(RBN == 256 || RBN == 128, "column block");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, cl = lane & 15;
  const int wm = wid / WN, wn = wid % WN;
  const int nsplit = p.nsplit;
  const int cb = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int ncols = EP == kEpSwiGLU ? 2 * p.w.seg_rows[0] : p.N;
  if (cb * RBN >= ncols) return;                 // the grid is laid out for 128-column blocks
  const int ncb128 = (ncols + kMgemmBN - 1) / kMgemmBN;
  f32x4_t tot[AF][4];
#pragma unroll
  for (int a = 0; a < AF; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) tot[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kpt = p.ks / pkt<Q4>();             // k-tiles per split
  pgemm_body<G, EP, Q4, RBN, 256, BM, true>(p, smem, ex, 0, cb, split * kpt, kpt, tot);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col = wn * 64 + t * 16 + cl;
    const int cb128 = cb * (RBN / kMgemmBN) + (col >> 7);
    if (cb128 >= ncb128) continue;
    float *mine = p.part + ((int64_t)cb128 * nsplit + split) * (BM * kMgemmBN) + (col & (kMgemmBN - 1));
#pragma unroll
    for (int a = 0; a < AF; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(wm * TM + a * 16 + 4 * qq + v) * kMgemmBN] = tot[a][t][v];
  }
}

template <int MB, int G, int EP>
__global__ __launch_bounds__(256) void mgemm_kernel(GemmParams p) {
  typedef MgemmShape<MB, G> S;
  constexpr int NT = S::NT, BN = S::BN, ROWS = S::ROWS, KS = S::KS;
  // LDS: the staged rows of the register path, or the ring (int4 layers;
  // bf16 for the LM head of 17 rows or more)
  constexpr int RB =
      EP == kEpLogits ? (MB >= 2 ? mgemm_ring_bytes<MB, G, false, kLogitsRbn>() : 0) : mgemm_ring_bytes<MB, G>();
  constexpr int SM = S::SMEM > RB ? S::SMEM : RB;
  __shared__ __align__(16) char smem[SM];
  __shared__ float xsg[ROWS * (KS / G)];
  __shared__ uint64_t rowkey[ROWS];
  __shared__ int last_flag;
  const MgemmLds L{reinterpret_cast<uint16_t *>(smem), xsg};
  float *Cs = reinterpret_cast<float *>(smem);

  const bool ex = p.path == kPathDevice ? layer_uses_exit(p.ctrl, p.layer) : p.path == kPathExit;
  const bool q4 = ex && p.exit_mode == RIVER_EXIT_INT4;
  if constexpr (EP == kEpLogits) {
    if constexpr (MB >= 2) {
      if (p.ring) {
        mgemm_ring<MB, G, EP, kLogitsRbn, false>(p, reinterpret_cast<uint4 *>(smem), false);
        return;
      }
    }
  } else {
    if (q4 && p.ring) {
      if constexpr (MB >= 2) {
        if (p.ring == 128) {
          mgemm_ring<MB, G, EP, 128>(p, reinterpret_cast<uint4 *>(smem), ex);
          return;
        }
      }
      mgemm_ring<MB, G, EP, 256>(p, reinterpret_cast<uint4 *>(smem), ex);
      return;
    }
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, cl = lane & 15;
  const int split = blockIdx.x % p.nsplit, colblk = blockIdx.x / p.nsplit;
  const int kbeg = split * p.ks;
  const int kend = min(p.K, kbeg + p.ks);

  f32x4_t tot[MB][NT];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) tot[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (q4) mgemm_body<MB, G, EP, true>(p, L, ex, colblk, kbeg, kend, tot);
  else mgemm_body<MB, G, EP, false>(p, L, ex, colblk, kbeg, kend, tot);

  if (p.nsplit > 1) {
    // partial tile straight from the accumulators, [ROWS][BN] row-major
    float *mine = p.part + ((int64_t)colblk * p.nsplit + split) * (ROWS * BN);
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          mine[(a * 16 + 4 * qq + v) * BN + wid * (NT * 16) + t * 16 + cl] = tot[a][t][v];
    return;
  }

  // ---- results to LDS (the slab buffer is reused)
  __syncthreads();
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        Cs[(a * 16 + 4 * qq + v) * (BN + 1) + wid * (NT * 16) + t * 16 + cl] = tot[a][t][v];
  __syncthreads();

  if constexpr (EP == kEpLogits) {
    logits_epilogue<ROWS, BN>(p, Cs, 0, colblk, rowkey, &last_flag);
  } else {
    tile_epilogue<EP, BN>(p, Cs, BN + 1, ROWS, 0, colblk);
  }
}

// Split-K sum of the batched-row GEMM and its epilogue: workgroup (column
// block, group of 8 rows) adds the partial tiles of the splits in order.
constexpr int kReduceRows = 8;
template <int MB, int EP>
__global__ __launch_bounds__(256) void mgemm_reduce_kernel(GemmParams p) {
  static_assert(EP != kEpLogits, "the LM head has its own reduce kernel");
  constexpr int BN = kMgemmBN, ROWS = MB * 16, RG = kReduceRows;
  __shared__ float Cs[RG * (BN + 1)];
  const int colblk = blockIdx.x / (ROWS / RG), rg = blockIdx.x % (ROWS / RG);
  const int i4 = threadIdx.x;                       // RG * BN / 4 == 256 float4
  const int r = (4 * i4) / BN, j = (4 * i4) % BN;
  const float *src = p.part + (int64_t)colblk * p.nsplit * (ROWS * BN) + (rg * RG + r) * BN + j;
  float4 v = *reinterpret_cast<const float4 *>(src);
#pragma unroll 4
  for (int sp = 1; sp < p.nsplit; ++sp) {
    const float4 t = *reinterpret_cast<const float4 *>(src + (int64_t)sp * (ROWS * BN));
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
  }
  float *c = Cs + r * (BN + 1) + j;
  c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
  __syncthreads();
  tile_epilogue<EP, BN>(p, Cs, BN + 1, RG, rg * RG, colblk);
}

// The same for the LM head, kLogitsBlocks column blocks per workgroup: the
// per-row maxima go out once per workgroup, so a vocabulary of ~1,000 column
// blocks makes 1/kLogitsBlocks of the agent-scope atomics and arrivals (each
// of which serialises on its address) that one workgroup per block would.
constexpr int kLogitsBlocks = 8;
template <int MB>
__global__ __launch_bounds__(256) void mgemm_reduce_logits_kernel(GemmParams p) {
  constexpr int BN = kMgemmBN, ROWS = MB * 16, RG = kReduceRows, C = kLogitsBlocks;
  __shared__ uint64_t rowkey[RG];
  __shared__ int last_flag;
  const int ncolblk = (p.N + BN - 1) / BN;
  const int cg = blockIdx.x / (ROWS / RG), rg = blockIdx.x % (ROWS / RG);
  const int i4 = threadIdx.x;                       // RG * BN / 4 == 256 float4
  const int r = (4 * i4) / BN, j = (4 * i4) % BN, m = rg * RG + r;
  if (threadIdx.x < RG) rowkey[threadIdx.x] = 0;
  // C column blocks of this row group: every split of all of them is loaded
  // before the sums are used (plain loads, C independent streams per thread)
  float4 v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int cb = min(cg * C + c, ncolblk - 1);
    v[c] = *reinterpret_cast<const float4 *>(p.part + (int64_t)cb * p.nsplit * (ROWS * BN) + r * BN +
                                             rg * RG * BN + j);
  }
  for (int sp = 1; sp < p.nsplit; ++sp) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int cb = min(cg * C + c, ncolblk - 1);
      const float4 t = *reinterpret_cast<const float4 *>(
          p.part + ((int64_t)cb * p.nsplit + sp) * (ROWS * BN) + r * BN + rg * RG * BN + j);
      v[c].x += t.x; v[c].y += t.y; v[c].z += t.z; v[c].w += t.w;
    }
  }
  uint64_t best = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int cb = cg * C + c;
    const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = cb * BN + j + q;
      if (cb >= ncolblk || m >= p.M || n >= p.N) continue;
      if (p.logits) p.logits[(int64_t)m * p.vocab + n] = e[q];
      const uint64_t key = logit_key(e[q], n);
      best = key > best ? key : best;
    }
  }
  __syncthreads();   // rowkey cleared
  if (best) __hip_atomic_fetch_max(&rowkey[r], best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();
  logits_finish<RG>(p, rg * RG, rowkey, &last_flag);
}

MgemmPlan mgemm_plan(int M, int ncols, int K, bool allow_split) {
  MgemmPlan pl{};
  pl.mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  pl.ncolblk = (ncols + kMgemmBN - 1) / kMgemmBN;
  const int KS = pl.mb == 1 ? 2048 : pl.mb == 2 ? 1024 : 512;
  // fewest splits the LDS allows (each split adds a partial tile of
  // rows x 128 fp32 per column block); more while the grid is short of one
  // workgroup per CU (256 on this chip)
  int ns = (K + KS - 1) / KS;
  if (allow_split)
    while (pl.ncolblk * ns < 256 && K / (ns * 2) >= 256 && (K / (ns * 2)) % 128 == 0) ns *= 2;
  int ks = (K + ns - 1) / ns;
  ks = (ks + 127) / 128 * 128;
  pl.ks = std::min(ks, K);
  pl.nsplit = (K + pl.ks - 1) / pl.ks;
  return pl;
}
MgemmPlan mgemm_plan(int M, int ncols, int K) { return mgemm_plan(M, ncols, K, true); }

// Plan of a linear whose layer may run on its int4 copy: the int4 path goes
// through the copy ring in 256-column blocks, and K is split into whole
// k-tiles of 128, at least two splits, the fewest that give a workgroup per CU
// (256 on this chip); the register path of the bf16 layers takes the same
// split (the weight form is chosen on the device), so a split also stays
// within the rows it can stage.
static bool mgemm_ring_ok(Epilogue ep, const GemmParams &p) {
  return ep != kEpLogits && p.layer >= 0 && p.exit_mode == RIVER_EXIT_INT4 &&
         (p.path == kPathDevice || p.path == kPathExit) && p.K % (2 * pkt<true>()) == 0;
}
static MgemmPlan mgemm_ring_plan_bn(int M, int ncols, int K, int rbn) {
  MgemmPlan pl{};
  pl.mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  pl.ncolblk = (ncols + kMgemmBN - 1) / kMgemmBN;
  pl.rbn = rbn;
  const int KS = pl.mb == 1 ? 2048 : pl.mb == 2 ? 1024 : 512;
  const int nt = K / pkt<true>(), ncb = (ncols + rbn - 1) / rbn;
  constexpr int kMinKs = 512;                   // K columns per split at least (measured best)
  int best = 0;
  for (int d = 2; d <= nt; ++d) {
    if (nt % d != 0 || K / d > KS) continue;
    if (best && K / d < kMinKs) break;
    best = d;
    if (ncb * d >= 256) break;
  }
  pl.nsplit = best;
  pl.ks = best ? K / best : 0;
  return pl;
}
// 256-column blocks, or 128-column ones (from 32 rows) where the 256-column
// plan fills at most half the CUs: at 32 rows the o projection (4,096 x
// 4,096) 13.4 -> 11.7 us, while q|k|v (192 workgroups) and down (256) were
// slower with 128 (the rows tile read by twice the workgroups, each unpacked
// B operand feeding half the MFMAs)
static MgemmPlan mgemm_ring_plan(int M, int ncols, int K) {
  MgemmPlan pl = mgemm_ring_plan_bn(M, ncols, K, 256);
  if (pl.mb >= 2 && pl.nsplit && ((ncols + 255) / 256) * pl.nsplit <= 128) {
    const MgemmPlan narrow = mgemm_ring_plan_bn(M, ncols, K, 128);
    if (narrow.nsplit >= 2) pl = narrow;
  }
  return pl;
}

// The LM head from 17 rows on (bf16 weights through the ring): 256-column
// blocks, K in two halves of whole 64-column k-tiles.  With K >= 2048 the
// register path's plan for the same rows splits K at least twice as often, so
// the workspace sized for that plan holds these partials.
static bool mgemm_logits_ring_ok(Epilogue ep, const GemmParams &p) {
  return ep == kEpLogits && p.M > 16 && p.K >= 2048 && p.K % (2 * pkt<false>()) == 0;
}
static MgemmPlan mgemm_logits_ring_plan(int M, int ncols, int K) {
  MgemmPlan pl{};
  pl.mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  pl.ncolblk = (ncols + kMgemmBN - 1) / kMgemmBN;
  pl.rbn = kLogitsRbn;
  pl.nsplit = 2;
  pl.ks = K / 2;
  return pl;
}

int64_t mgemm_part_floats(const MgemmPlan &pl) {
  return pl.nsplit > 1 ? (int64_t)pl.ncolblk * pl.nsplit * (pl.mb * 16) * kMgemmBN : 0;
}

int64_t mgemm_part_floats_max(int M, int ncols, int K) {
  int64_t f = mgemm_part_floats(mgemm_plan(M, ncols, K));
  if (K % (2 * pkt<true>()) == 0) f = std::max(f, mgemm_part_floats(mgemm_ring_plan(M, ncols, K)));
  return f;
}

template <int MB>
static hipError_t mgemm_reduce(Epilogue ep, const GemmParams &p, int grid, hipStream_t s) {
  switch (ep) {
    case kEpQKV: return launch_1(mgemm_reduce_kernel<MB, kEpQKV>, dim3(grid), dim3(256), p, s);
    case kEpResid: return launch_1(mgemm_reduce_kernel<MB, kEpResid>, dim3(grid), dim3(256), p, s);
    case kEpSwiGLU: return launch_1(mgemm_reduce_kernel<MB, kEpSwiGLU>, dim3(grid), dim3(256), p, s);
    case kEpPlain: return launch_1(mgemm_reduce_kernel<MB, kEpPlain>, dim3(grid), dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MB, int G>
static hipError_t mgemm_launch_g(Epilogue ep, const GemmParams &p, int grid, hipStream_t s) {
  switch (ep) {
    case kEpQKV: return launch_1(mgemm_kernel<MB, G, kEpQKV>, dim3(grid), dim3(256), p, s);
    case kEpResid: return launch_1(mgemm_kernel<MB, G, kEpResid>, dim3(grid), dim3(256), p, s);
    case kEpSwiGLU: return launch_1(mgemm_kernel<MB, G, kEpSwiGLU>, dim3(grid), dim3(256), p, s);
    case kEpLogits: return launch_1(mgemm_kernel<MB, G, kEpLogits>, dim3(grid), dim3(256), p, s);
    case kEpPlain: return launch_1(mgemm_kernel<MB, G, kEpPlain>, dim3(grid), dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MB>
static hipError_t mgemm_launch_mb(Epilogue ep, const GemmParams &p, int ncolblk, hipStream_t s) {
  hipError_t e;
  switch (p.G) {
    case 64: e = mgemm_launch_g<MB, 64>(ep, p, ncolblk * p.nsplit, s); break;
    case 128: e = mgemm_launch_g<MB, 128>(ep, p, ncolblk * p.nsplit, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || p.nsplit == 1) return e;
  static_assert(kReduceRows * kMgemmBN / 4 == 256, "one float4 per thread");
  if (ep == kEpLogits)
    return launch_1(mgemm_reduce_logits_kernel<MB>,
                    dim3(((ncolblk + kLogitsBlocks - 1) / kLogitsBlocks) * (MB * 16 / kReduceRows)), dim3(256),
                    p, s);
  return mgemm_reduce<MB>(ep, p, ncolblk * (MB * 16 / kReduceRows), s);
}

hipError_t launch_mgemm(Epilogue ep, const GemmParams &p, hipStream_t s) {
  if (p.M < 1 || p.M > 64 || p.K % p.G || (p.G != 64 && p.G != 128)) return hipErrorInvalidValue;
  const int ncols = ep == kEpSwiGLU ? 2 * p.w.seg_rows[0] : p.N;
  const bool lring = mgemm_logits_ring_ok(ep, p);
  const bool ring = lring || mgemm_ring_ok(ep, p);
  const MgemmPlan pl = lring  ? mgemm_logits_ring_plan(p.M, ncols, p.K)
                       : ring ? mgemm_ring_plan(p.M, ncols, p.K)
                              : mgemm_plan(p.M, ncols, p.K, ep != kEpLogits);
  if (ring && pl.nsplit < 2) return hipErrorInvalidValue;
  if (pl.nsplit > 1 && (!p.part || mgemm_part_floats(pl) > p.part_cap)) return hipErrorInvalidValue;
  // (the register path stages a whole split of the rows; the LM head's ring
  // never takes that path)
  if (!lring && pl.ks > (pl.mb == 1 ? 2048 : pl.mb == 2 ? 1024 : 512)) return hipErrorInvalidValue;
  GemmParams q = p;
  q.nsplit = pl.nsplit;
  q.ks = pl.ks;
  q.ring = ring ? pl.rbn : 0;
  switch (pl.mb) {
    case 1: return mgemm_launch_mb<1>(ep, q, pl.ncolblk, s);
    case 2: return mgemm_launch_mb<2>(ep, q, pl.ncolblk, s);
    default: return mgemm_launch_mb<4>(ep, q, pl.ncolblk, s);
  }
}


template <int G, int EP, int BN, int NTH = kPThreads, int BM = kPBM>
__global__ __launch_bounds__(NTH, 1) void pgemm_kernel(GemmParams p, int nrowblk, int ncolblk) {
  // three stages of rows and weights (and int4 scale/zero words); the
  // results reuse them
  __shared__ __align__(16) uint4 smem[psmem_slots<G, BN, NTH, BM>()];
  constexpr int TM = ptm<BN, NTH, BM>(), AF = TM / 16;
  bool ex = p.path == kPathDevice ? layer_uses_exit(p.ctrl, p.layer) : p.path == kPathExit;
  // grouped order: kPGroupRows row blocks share the weights of each column block
  const int per_group = kPGroupRows * ncolblk;
  const int grp = blockIdx.x / per_group;
  const int first = grp * kPGroupRows;
  const int gm = min(nrowblk - first, kPGroupRows);
  const int in_grp = blockIdx.x - grp * per_group;
  const int rowblk = first + in_grp % gm, colblk = in_grp / gm;
  if (past_exit_skip<EP, BN>(p, colblk, ex)) return;   // (comparators)
  const bool q4 = ex && p.exit_mode == RIVER_EXIT_INT4;

  f32x4_t tot[AF][4];
#pragma unroll
  for (int a = 0; a < AF; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) tot[a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // K split over gridDim.y in whole 128-column units (one int4 k-tile, two
  // bf16 ones), so that both weight forms split at the same columns
  const int nsp = gridDim.y, sp = blockIdx.y;
  const int units = p.K / pkt<true>(), u0 = units * sp / nsp, u1 = units * (sp + 1) / nsp;
  if (q4) pgemm_body<G, EP, true, BN, NTH, BM>(p, smem, ex, rowblk, colblk, u0, u1 - u0, tot);
  else pgemm_body<G, EP, false, BN, NTH, BM>(p, smem, ex, rowblk, colblk, 2 * u0, 2 * (u1 - u0), tot);

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int qq = lane >> 4, cl = lane & 15;
  const int wm = wid / pwn<BN>(), wn = wid % pwn<BN>();
  if constexpr (EP == kEpResid) {
    if (nsp > 1) {
      // partial tile of split sp: part[sp][row][col], rows of whole blocks;
      // pgemm_reduce_kernel adds the splits and runs the epilogue
      float *part = p.part + (int64_t)sp * nrowblk * BM * p.N;
#pragma unroll
      for (int a = 0; a < AF; ++a)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = colblk * BN + wn * 64 + t * 16 + cl;
          if (col < p.N) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              part[((int64_t)rowblk * BM + wm * TM + a * 16 + 4 * qq + v) * p.N + col] = tot[a][t][v];
          }
        }
      return;
    }
  }

  // results through LDS (the body ends with a barrier and no copy in flight)
  float *Cs = reinterpret_cast<float *>(smem);
  static_assert(BM * (BN + 1) * 4 <= psmem_slots<G, BN, NTH, BM>() * 16, "the results fit the buffers");
#pragma unroll
  for (int a = 0; a < AF; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        Cs[(wm * TM + a * 16 + 4 * qq + v) * (BN + 1) + wn * 64 + t * 16 + cl] = tot[a][t][v];
  __syncthreads();
  tile_epilogue<EP, BN, NTH>(p, Cs, BN + 1, BM, (int64_t)rowblk * BM, colblk);
}

// Split-K sum of the prefill GEMM (kEpResid) and its epilogue: workgroup
// (128-column block, group of 8 rows) adds the partial tiles in split order.
constexpr int kPRedRows = 8;
template <int EP>
__global__ __launch_bounds__(256) void pgemm_reduce_kernel(GemmParams p, int mrows, int nsplit) {
  constexpr int BN = 128, RG = kPRedRows;
  static_assert(RG * BN / 4 == 256, "one float4 per thread");
  __shared__ float Cs[RG * (BN + 1)];
  // (comparators: the GEMM passed the residual stream through already)
  if (past_exit_action(p.ctrl, p.layer, p.path) != kRun) return;
  const int ncb = (p.N + BN - 1) / BN;
  const int colblk = blockIdx.x % ncb, rg = blockIdx.x / ncb;
  const int r = threadIdx.x / (BN / 4), j = 4 * (threadIdx.x % (BN / 4));
  const int col = colblk * BN + j;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < p.N) {
    const float *src = p.part + ((int64_t)rg * RG + r) * p.N + col;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float4 t = *reinterpret_cast<const float4 *>(src + (int64_t)sp * mrows * p.N);
      v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
    }
  }
  float *c = Cs + r * (BN + 1) + j;
  c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
  __syncthreads();
  tile_epilogue<EP, BN>(p, Cs, BN + 1, RG, (int64_t)rg * RG, colblk);
}

template <int G, int BN, int NTH = kPThreads, int BM = kPBM>
static hipError_t pgemm_launch_gb(Epilogue ep, const GemmParams &p, hipStream_t s, int nsplit = 1) {
  const int ncols = ep == kEpSwiGLU ? 2 * p.w.seg_rows[0] : p.N;
  int nrowblk = (p.M + BM - 1) / BM, ncolblk = (ncols + BN - 1) / BN;
  GemmParams q = p;
  void *args[] = {&q, &nrowblk, &ncolblk};
  const dim3 grid((unsigned)(nrowblk * ncolblk), (unsigned)nsplit);
  const void *fn;
  switch (ep) {
    case kEpQKV: fn = reinterpret_cast<const void *>(pgemm_kernel<G, kEpQKV, BN, NTH, BM>); break;
    case kEpSwiGLU: fn = reinterpret_cast<const void *>(pgemm_kernel<G, kEpSwiGLU, BN, NTH, BM>); break;
    case kEpResid: fn = reinterpret_cast<const void *>(pgemm_kernel<G, kEpResid, BN, NTH, BM>); break;
    case kEpPlain: fn = reinterpret_cast<const void *>(pgemm_kernel<G, kEpPlain, BN, NTH, BM>); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = launch_kernel(fn, grid, dim3(NTH), args, 0, s);
  if (e != hipSuccess || nsplit == 1) return e;
  // (only kEpResid launches split K)
  int mrows = nrowblk * BM, ns = nsplit;
  void *rargs[] = {&q, &mrows, &ns};
  const dim3 rgrid((unsigned)(((p.N + 127) / 128) * (mrows / kPRedRows)));
  return launch_kernel(reinterpret_cast<const void *>(pgemm_reduce_kernel<kEpResid>), rgrid, dim3(256), rargs, 0, s);
}

// 256-column blocks (64 x 64 per wavefront: half the int4 unpacking per
// MFMA of 128-column blocks) once there are enough rows to fill the chip
// with them; 128-column blocks for shorter prompts.  Up to kPSmallRows rows a
// layer that may run on its int4 copy takes 64-row x 128-column tiles of 256
// threads instead (twice the workgroups, two per CU): at 256 and 512 rows
// the int4 GEMMs ran 16-17% faster so, while bf16 weights, read twice as often
// per flop, ran 4-17% slower (and from 1,024 rows int4 gained <= 6%, bf16 lost
// up to 27%), so a layer known to run on its backbone (a backbone path, or a
// pending-row pass) keeps the larger tile.  Where even the 64-row tiles leave
// fewer workgroups than CUs (256 on this chip), 32-row tiles double them: on
// the 1B shape at 256 rows (q|k|v, o and down: 96, 64 and 64 workgroups) the
// int4 prefill GEMMs 179 -> 220 TFLOP/s; on the 8B shape at 512 rows (256 or
// more everywhere) 32-row tiles for the linears under 512 workgroups were
// slower (517-524 -> 502-506).
constexpr int kPSmallRows = 512;
template <int G>
static hipError_t pgemm_launch_g(Epilogue ep, const GemmParams &p, hipStream_t s) {
  if (p.M >= kPWideRows) return pgemm_launch_gb<G, 256>(ep, p, s);
  // (a pending-row pass runs the backbone, as a backbone path does)
  const bool may_q4 =
      p.exit_mode == RIVER_EXIT_INT4 && p.layer >= 0 && (p.path == kPathDevice || p.path == kPathExit);
  if (p.M <= kPSmallRows && may_q4) {
    const int ncols = ep == kEpSwiGLU ? 2 * p.w.seg_rows[0] : p.N;
    const int wgs = ((p.M + 63) / 64) * ((ncols + 127) / 128);
    if (wgs < 256) return pgemm_launch_gb<G, 128, 256, 32>(ep, p, s);
    // o and down with fewer than two workgroups per CU: K in two halves,
    // partial tiles in the caller's buffer, added up by a second kernel
    const int64_t part = 2 * (int64_t)((p.M + 63) / 64) * 64 * p.N;
    if (ep == kEpResid && wgs < 512 && p.part && part <= p.part_cap && p.N % 4 == 0 &&
        (p.K / pkt<true>()) >= 2)
      return pgemm_launch_gb<G, 128, 256, 64>(ep, p, s, 2);
    return pgemm_launch_gb<G, 128, 256, 64>(ep, p, s);
  }
  return pgemm_launch_gb<G, 128>(ep, p, s);
}

bool pgemm_fits(int K, int G) {
  // K in whole k-tiles of either weight form
  return (G == 64 || G == 128) && K % pkt<true>() == 0;
}

hipError_t launch_pgemm(Epilogue ep, const GemmParams &p, hipStream_t s) {
  if (!pgemm_fits(p.K, p.G)) return hipErrorInvalidValue;
  return p.G == 64 ? pgemm_launch_g<64>(ep, p, s) : pgemm_launch_g<128>(ep, p, s);
}

}  // namespace river
