// Prefill kernels for gfx950 (and the batched-decode linears): RMSNorm over
// rows, an MFMA bf16 GEMM whose weight operand is either bf16 or the int4 exit
// copy dequantised on the fly, causal GQA attention over the prompt, and the
// sequence-level exit test (one decision for all B*T prompt rows).
//
// Method: "River-LLM: Large Language Model Seamless Exit Based on KV Share",
// section 5: prefill exits at the sequence level so that every prompt token
// leaves at the same layer and the prompt stays one parallel pass.
#include "device_common.h"

namespace river {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ===========================================================================
// RMSNorm rows: x[r] = bf16(h[r] / sqrt(mean(h[r]^2) + eps) * gain); one
// wavefront per row.
// ===========================================================================
__global__ __launch_bounds__(256) void rows_norm_kernel(RowsNormParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const float *h = p.h + r * p.d;
  float ss = 0.f;
  for (int k = lane * 4; k < p.d; k += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(h + k);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)p.d + p.eps);
  uint16_t *x = p.x + r * p.d;
  for (int k = lane * 4; k < p.d; k += 256) {
    const float4 v = *reinterpret_cast<const float4 *>(h + k);
    const uint2 g = *reinterpret_cast<const uint2 *>(p.gain + k);
    uint2 o;
    o.x = pack_bf2(v.x * rs * bf_lo(g.x), v.y * rs * bf_hi(g.x));
    o.y = pack_bf2(v.z * rs * bf_lo(g.y), v.w * rs * bf_hi(g.y));
    *reinterpret_cast<uint2 *>(x + k) = o;
  }
}

hipError_t launch_rows_norm(const RowsNormParams &p, hipStream_t s) {
  const int64_t blocks = (p.rows + 3) / 4;
  return launch_1(rows_norm_kernel, dim3((unsigned)blocks), dim3(256), p, s);
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

template <int BM, int BN, int EP>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int LDSK = kBK + kLdsPad;
  constexpr int TM = BM / 32, TN = BN / 32;   // 16x16 tiles per wave
  __shared__ __align__(16) uint16_t As[BM][LDSK];
  __shared__ __align__(16) uint16_t Bs[BN][LDSK];
  __shared__ float Cs[BM][BN + 1];
  __shared__ uint32_t szs[BN];
  __shared__ float xsg[BM];

  const bool ex = p.path == kPathDevice ? layer_uses_exit(p.ctrl, p.layer) : p.path == kPathExit;
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
        // word i covers columns 8i..8i+7; column 8i+j sits in bits 4j..4j+3
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t o[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t c0 = (wd[i] >> (8 * jj)) & 0xF;
            const uint32_t c1 = (wd[i] >> (8 * jj + 4)) & 0xF;
            o[jj] = (0x4300u | c0) | ((0x4300u | c1) << 16);
          }
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

  // ---- epilogues
  if constexpr (EP == kEpQKV) {
    const int half = p.Dh >> 1;
    for (int idx = tid; idx < BM * (BN / 2); idx += 256) {
      const int r = idx / (BN / 2), pp = idx % (BN / 2);
      const int64_t m = m0 + r;
      const int L0 = blockIdx.y * BN + 2 * pp;
      if (m >= p.M || L0 >= p.N) continue;
      int b, t;
      if (p.T > 0) { b = (int)(m / p.T); t = (int)(m % p.T); }
      else { b = (int)m; t = p.ctrl->pos; }
      const int P = L0 >> 1;
      const int hh = P / half, i = P % half;
      float y0 = Cs[r][2 * pp], y1 = Cs[r][2 * pp + 1];
      if (hh < p.Hq + p.Hkv) {
        const double ang = (double)t * pow((double)p.rope_theta, -2.0 * i / (double)p.Dh);
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float c = (float)cs, s = (float)sn;
        const float a0 = y0 * c - y1 * s;
        const float a1 = y1 * c + y0 * s;
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
    for (int idx = tid; idx < BM * hw; idx += 256) {
      const int r = idx / hw, jj = idx % hw;
      const int64_t m = m0 + r;
      const int n = blockIdx.y * hw + jj;
      if (m >= p.M || n >= p.w.seg_rows[0]) continue;
      const float gt = Cs[r][jj], up = Cs[r][hw + jj];
      p.u_out[m * p.w.seg_rows[0] + n] = f2bf(gt / (1.0f + expf(-gt)) * up);
    }
  } else if constexpr (EP == kEpPlain) {
    for (int idx = tid; idx < BM * BN; idx += 256) {
      const int r = idx / BN, j = idx % BN;
      const int64_t m = m0 + r;
      const int n = blockIdx.y * BN + j;
      if (m < p.M && n < p.N) p.y_out[m * p.y_stride + n] = Cs[r][j];
    }
  } else {  // residual
    for (int idx = tid; idx < BM * BN; idx += 256) {
      const int r = idx / BN, j = idx % BN;
      const int64_t m = m0 + r;
      const int n = blockIdx.y * BN + j;
      if (m >= p.M || n >= p.N) continue;
      const int64_t o = m * p.h_io_stride + n;
      p.h_out[o] = p.h_in[o] + Cs[r][j];
    }
  }
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
//   each owning Dh/4 of the head dimension; K/V tiles of 32 positions staged
//   in LDS.  Scores q.k / sqrt(Dh), fp32 softmax.
// ===========================================================================
template <int DH>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillParams p) {
  constexpr int SL = DH / 4;    // elements per thread
  constexpr int KT = 32;        // keys per tile
  __shared__ __align__(16) uint16_t Ks[KT][DH];
  __shared__ __align__(16) uint16_t Vs[KT][DH];
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (p.Hq / p.Hkv);
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int t = qb * 64 + r;
  const bool live = t < p.T;
  const int64_t qrow = (int64_t)b * p.T + t;
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
  const int kend = min(p.T, qb * 64 + 64);  // keys needed by this block
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
      const bool ok = live && (k0 + j) <= t;
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

hipError_t launch_attn_prefill(const AttnPrefillParams &p, hipStream_t s) {
  dim3 grid((p.T + 63) / 64, p.Hq, p.B);
  switch (p.Dh) {
    case 64: return launch_1(attn_prefill_kernel<64>, grid, dim3(256), p, s);
    case 128: return launch_1(attn_prefill_kernel<128>, grid, dim3(256), p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace river
