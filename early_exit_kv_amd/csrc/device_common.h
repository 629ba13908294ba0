// Device helpers shared by the gfx950 kernels: bf16 <-> fp32, wavefront
// reductions, agent-scope ordering for the last-workgroup pattern.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "river_internal.h"

namespace river {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// N consecutive 32-bit words as one load
// LDS pointer type (for the LDS byte address of a __shared__ object)
typedef __attribute__((address_space(3))) void *lds_ptr_t;
// compile-time index (of a register buffer, a ring slot, a variant), passed
// to generic lambdas
template <int N> struct Buf { static constexpr int value = N; };
template <int N_> struct WordsT;
template <> struct WordsT<1> { typedef uint32_t T; };
template <> struct WordsT<2> { typedef v2u T; };
template <> struct WordsT<4> { typedef v4u T; };

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs held in 32-bit words
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// DPP cross-lane moves (no LDS traffic).  row_ror:n rotates within each row
// of 16 lanes; quad_perm permutes within each group of 4; half_mirror reverses
// each half-row of 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppRor1 = 0x121, kDppRor2 = 0x122, kDppRor4 = 0x124, kDppRor8 = 0x128;
constexpr int kDppHalfMirror = 0x141, kDppXor1 = 0xB1, kDppXor2 = 0x4E;

// all-reduce within aligned groups of 16 (sum16) or 8 (sum8) lanes
__device__ __forceinline__ float sum16(float v) {
  v += dpp<kDppRor8>(v);
  v += dpp<kDppRor4>(v);
  v += dpp<kDppRor2>(v);
  v += dpp<kDppRor1>(v);
  return v;
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<kDppRor8>(v));
  v = fmaxf(v, dpp<kDppRor4>(v));
  v = fmaxf(v, dpp<kDppRor2>(v));
  v = fmaxf(v, dpp<kDppRor1>(v));
  return v;
}
// wavefront sum, returned as a wave-uniform value
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v = sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// sum over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide sum over blockDim.x threads (a multiple of 64, at most 1024).
// `red` holds at least blockDim.x/64 floats.  All threads get the result.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) t += red[i];  // fixed order: deterministic
  return t;
}
__device__ __forceinline__ float block_min(float v, float *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = red[0];
  const int nw = blockDim.x >> 6;
  for (int i = 1; i < nw; ++i) t = fminf(t, red[i]);
  return t;
}

// Last-workgroup hand-off: every workgroup publishes its results, then thread
// 0 counts itself in; the workgroup that brings the count to `total` resets
// the counter and may read what the others published.
//
// Contract: every value handed from one workgroup to another inside a kernel
// is written with st_coherent and read with ld_coherent (relaxed agent-scope
// atomics, which are coherent across the XCDs on their own: they are not kept
// dirty in one XCD's L2).  The counter itself is a relaxed atomic too; there
// is no release/acquire fence (on gfx950 such fences write back or invalidate
// the whole L2), so a plain store or load of handed-over data would NOT be
// ordered by this hand-off.  Ordering comes from each thread waiting for its
// own coherent stores to complete (s_waitcnt vmcnt(0), also a compiler
// barrier) before the workgroup barrier, after which thread 0 counts the
// workgroup in.
__device__ __forceinline__ void st_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bool arrive_last(uint32_t *counter, uint32_t total, int *smem_flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == total - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *smem_flag = last;
  }
  __syncthreads();
  asm volatile("" ::: "memory");
  return *smem_flag != 0;
}

// int4 codes of one 32-bit word (byte i: column i in the low nibble, column
// i+4 in the high nibble) as the four bf16 pairs (128+q_a, 128+q_b) of the
// columns (0,1) (2,3) (4,5) (6,7): the byte permute places each code under a
// 0x43 byte, and 0x43nn is the bf16 value 128 + nn for nn < 16
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t (&pr)[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  pr[0] = __builtin_amdgcn_perm(0x43434343u, lo, 0x05010400u);
  pr[1] = __builtin_amdgcn_perm(0x43434343u, lo, 0x05030402u);
  pr[2] = __builtin_amdgcn_perm(0x43434343u, hi, 0x05010400u);
  pr[3] = __builtin_amdgcn_perm(0x43434343u, hi, 0x05030402u);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Exit choice of a layer, read at the start of every kernel of that layer.
__device__ __forceinline__ bool layer_uses_exit(const Control *c, int layer) {
  if (layer < 0) return false;
  const int fe = c->force_E;
  if (fe >= 0) return layer >= fe;
  return c->flag != 0;
}

// Under the prior-art comparators (KvStrategy other than the river) a layer
// at or past the exit does not run as an exit layer: what its kernels do.
enum PastExit { kRun = 0, kSkip = 1, kKvOnly = 2 };
__device__ __forceinline__ int past_exit_action(const Control *c, int layer, int path) {
  if (layer < 0) return kRun;
  const int st = c->strategy;
  if (st == kStratRiver) return kRun;
  const bool past = (path == kPathDevice || path == kPathPending) ? layer_uses_exit(c, layer)
                                                                  : path == kPathExit;
  if (!past) return kRun;
  return st == kStratPropagate ? kKvOnly : kSkip;
}

// Monotone map of fp32 to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace river
