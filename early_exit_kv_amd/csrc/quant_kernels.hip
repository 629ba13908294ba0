// Exit-layer construction on gfx950: copy + 4-bit group quantisation of one
// linear matrix ("River-LLM: Large Language Model Seamless Exit Based on KV
// Share", section 3: exit layers are copies of each layer quantised to W4A16,
// made without training).
//
// Per (row, group of G columns), float32 with every operation rounded on its
// own (IEEE division, no contraction) so that the codes are reproducible
// bit for bit:
//   s = bf16((hi - lo) / 15), s = 1 if that is 0;  z = bf16(-lo / s);
//   code = clamp(round_half_even(w / s + z), 0, 15).
// One thread packs one 32-bit word (8 columns: byte i holds column i in its
// low nibble and column i+4 in its high nibble, so that a byte permute turns
// the word into the bf16 pairs of columns (0,1) (2,3) (4,5) (6,7) in order);
// the G/8 threads of a group sit
// in adjacent lanes and find the group's min and max with lane shuffles.
#include "device_common.h"

#pragma clang fp contract(off)

namespace river {

__device__ __forceinline__ float bf16_round(float f) { return bf2f(f2bf(f)); }

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ w, int64_t words,
                                                       int KW, int G, uint32_t *__restrict__ codes,
                                                       uint32_t *__restrict__ sz) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < words;
  const int gw = G / 8;  // threads (words) per group, a power of two <= 64
  float v[8];
  float lo = INFINITY, hi = -INFINITY;
  if (live) {
    const uint4 u = *reinterpret_cast<const uint4 *>(w + i * 8);
    v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
    v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
#pragma unroll
    for (int j = 0; j < 8; ++j) { lo = fminf(lo, v[j]); hi = fmaxf(hi, v[j]); }
  }
  for (int o = gw >> 1; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  if (!live) return;
  float s = bf16_round(__fdiv_rn(__fsub_rn(hi, lo), 15.0f));
  if (s == 0.0f) s = 1.0f;
  const float z = bf16_round(__fdiv_rn(-lo, s));
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q = rintf(__fadd_rn(__fdiv_rn(v[j], s), z));
    q = fminf(fmaxf(q, 0.0f), 15.0f);
    // byte i of the word: column 8w+i in the low nibble, column 8w+i+4 in the high one
    word |= (uint32_t)q << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
  }
  codes[i] = word;
  const int64_t row = i / KW;
  const int wi = (int)(i % KW);
  if (wi % gw == 0)
    sz[row * (KW / gw) + wi / gw] = (uint32_t)f2bf(s) | ((uint32_t)f2bf(z) << 16);
}

// ---------------------------------------------------------------------------
// The same quantiser followed by an HQQ-style refinement of the zero point
// (half-quadratic rounds; the l1 norm's soft threshold as the proximal step),
// per (row, group), float32 with every operation rounded on its own and
// zf = z to begin with:
//   q  = clamp(round_half_even(w / s + zf), 0, 15)
//   e  = w - (q - zf) s;   we = sign(e) max(|e| - 1/beta, 0)
//   zf = (sum over the group of q - (w - we) / s) / G;   beta = beta kappa
// The group sum is a fixed pairwise tree: the two halves of the group are
// added element-wise, then the halves of that, down to one value; with the
// group's 8-column words in G/8 adjacent lanes, the halves wider than a word
// are lane butterflies (xor G/16 .. 1) and the last three levels are inside
// a lane.  Every lane of the group then holds the same sum.  The scale keeps
// its min-max value, the zero is stored as bf16(zf), and the codes are taken
// with the stored scale and zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_hqq_kernel(const uint16_t *__restrict__ w, int64_t words,
                                                           int KW, int G, uint32_t *__restrict__ codes,
                                                           uint32_t *__restrict__ sz, int iters, float beta,
                                                           float kappa) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = i < words;
  const int gw = G / 8;  // lanes (words) per group, a power of two <= 64
  float v[8];
  float lo = INFINITY, hi = -INFINITY;
  if (live) {
    const uint4 u = *reinterpret_cast<const uint4 *>(w + i * 8);
    v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
    v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
#pragma unroll
    for (int j = 0; j < 8; ++j) { lo = fminf(lo, v[j]); hi = fmaxf(hi, v[j]); }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;   // (lanes past the end: inert, never stored)
  }
  for (int o = gw >> 1; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  float s = bf16_round(__fdiv_rn(__fsub_rn(hi, lo), 15.0f));
  if (!(s != 0.0f)) s = 1.0f;   // (also the inert lanes past the end, whose range is empty)
  float zf = bf16_round(__fdiv_rn(-lo, s));
  if (!live) zf = 0.0f;
  float b = beta;
  const float inv_g = 1.0f / (float)G;   // a power of two: exact
  for (int it = 0; it < iters; ++it) {
    const float thr = __fdiv_rn(1.0f, b);
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float q = rintf(__fadd_rn(__fdiv_rn(v[j], s), zf));
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      const float e = __fsub_rn(v[j], __fmul_rn(__fsub_rn(q, zf), s));
      const float m = fmaxf(__fsub_rn(fabsf(e), thr), 0.0f);
      const float we = e > 0.0f ? m : (e < 0.0f ? -m : 0.0f);
      t[j] = __fsub_rn(q, __fdiv_rn(__fsub_rn(v[j], we), s));
    }
    // tree sum: halves of G/16 words .. 1 word across lanes, then 4, 2, 1 columns
    for (int o = gw >> 1; o > 0; o >>= 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = __fadd_rn(t[j], __shfl_xor(t[j], o, 64));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = __fadd_rn(t[j], t[j + 4]);
    t[0] = __fadd_rn(t[0], t[2]);
    t[1] = __fadd_rn(t[1], t[3]);
    zf = __fmul_rn(__fadd_rn(t[0], t[1]), inv_g);
    b = __fmul_rn(b, kappa);
  }
  if (!live) return;
  const float z = bf16_round(zf);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q = rintf(__fadd_rn(__fdiv_rn(v[j], s), z));
    q = fminf(fmaxf(q, 0.0f), 15.0f);
    word |= (uint32_t)q << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
  }
  codes[i] = word;
  const int64_t row = i / KW;
  const int wi = (int)(i % KW);
  if (wi % gw == 0)
    sz[row * (KW / gw) + wi / gw] = (uint32_t)f2bf(s) | ((uint32_t)f2bf(z) << 16);
}

hipError_t launch_quantize_hqq(const uint16_t *w, int N, int K, int G, uint32_t *codes, uint32_t *sz,
                               int iters, float beta, float kappa, hipStream_t s) {
  if (G < 32 || G > 512 || (G & (G - 1)) || K % G || iters < 0) return hipErrorInvalidValue;
  const int64_t words = (int64_t)N * (K / 8);
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(quantize_hqq_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, words, K / 8, G,
                     codes, sz, iters, beta, kappa);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *w, int N, int K, int G, uint32_t *codes, uint32_t *sz,
                           hipStream_t s) {
  if (G < 32 || G > 512 || (G & (G - 1)) || K % G) return hipErrorInvalidValue;
  const int64_t words = (int64_t)N * (K / 8);
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, words, K / 8, G,
                     codes, sz);
  return hipGetLastError();
}

}  // namespace river
